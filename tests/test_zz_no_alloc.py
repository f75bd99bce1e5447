"""The allocation-free selection entry point (fp2_select_blocks_noalloc,
workspace in the library's static device array) against fp2_select_blocks
with a caller workspace, through the C ABI: two calls in a row, the second
smaller, each bit-identical to the regular call; and a call beyond the
static array's 16 MiB refused before anything is enqueued."""

import pytest
import torch

import block_sparse_long_scores_amd as fp2_mod
import synth

SCRATCH_BYTES = 16 << 20
FAKE = 0x1000  # non-NULL pointer that is never dereferenced by validation


def _regular_and_noalloc(fp2, p, q, k, v):
    """Both entry points on the same inputs, each into its own outputs
    (pre-filled with sentinels)."""
    B, Sq, Sk = q.shape[0], q.shape[1], k.shape[1]
    nqb, nkb = fp2.fp2_num_q_blocks(Sq, Sk, p.block_size), fp2.fp2_num_k_blocks(Sk, p.block_size)
    hkv, d = p.num_kv_heads, p.head_dim
    sh = torch.cuda.current_stream().cuda_stream
    res = []
    for noalloc in (False, True):
        idx = torch.full((B, hkv, nqb, nkb), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, hkv, nqb), -7, dtype=torch.int32, device="cuda")
        pk = torch.full((B, hkv, nkb, d), float("nan"), dtype=torch.float32, device="cuda")
        pv = torch.full_like(pk, float("nan"))
        if noalloc:
            st = fp2.fp2_select_blocks_noalloc(p, B, Sq, Sk, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               idx.data_ptr(), cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(), sh)
        else:
            ws = torch.empty(fp2.fp2_select_workspace_size(p, B, Sq, Sk), dtype=torch.uint8, device="cuda")
            st = fp2.fp2_select_blocks(p, B, Sq, Sk, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                       cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(), ws.data_ptr(), ws.numel(), sh)
        assert st == fp2.FP2_OK, fp2.last_error()
        res.append((idx, cnt, pk, pv))
    torch.cuda.synchronize()
    return res


def _assert_same(a, b):
    (i1, c1, k1, v1), (i2, c2, k2, v2) = a, b
    assert torch.equal(c1, c2)
    assert bool((c1 >= 1).all())
    B, H, nqb, _ = i1.shape
    for s in range(B):
        for h in range(H):
            for il in range(nqb):
                c = int(c1[s, h, il])
                assert torch.equal(i1[s, h, il, :c], i2[s, h, il, :c]), (s, h, il)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)


@pytest.mark.gpu
def test_noalloc_select_equals_workspace_select_twice(gpu):
    # call 1: batch 2, 4096 tokens, group-mean selection
    hq, hkv, d, b = 8, 2, 128, 128
    prs = [synth.make_problem("planted", 50 + s, 4096, hq, hkv, d, b) for s in range(2)]
    q = torch.stack([x.q for x in prs]).cuda()
    k = torch.stack([x.k for x in prs]).cuda()
    v = torch.stack([x.v for x in prs]).cuda()
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    print(f"[case] noalloc call 1: B=2 S=4096 hq={hq} hkv={hkv} scratch use "
          f"{gpu.fp2_select_workspace_size(p, 2, 4096, 4096)} bytes", flush=True)
    r1 = _regular_and_noalloc(gpu, p, q, k, v)
    _assert_same(*r1)
    # call 2, smaller: batch 1, a 700-row chunk over 1500 keys, d 64 / b 64, union selection
    hq, hkv, d, b = 8, 2, 64, 64
    pr = synth.make_problem("planted", 52, 1500, hq, hkv, d, b, seqlen_q=700)
    p = gpu.make_params(hq, hkv, d, b, tau=0.5, select_mode="union")
    print(f"[case] noalloc call 2: B=1 Sq=700 Sk=1500 union, scratch use "
          f"{gpu.fp2_select_workspace_size(p, 1, 700, 1500)} bytes", flush=True)
    r2 = _regular_and_noalloc(gpu, p, pr.q[None].cuda(), pr.k[None].cuda(), pr.v[None].cuda())
    _assert_same(*r2)
    # and the first problem once more after the smaller one: still identical
    p = gpu.make_params(8, 2, 128, 128, tau=0.8)
    r3 = _regular_and_noalloc(gpu, p, q, k, v)
    _assert_same(*r3)
    _assert_same(r1[0], r3[1])


def test_noalloc_refuses_calls_beyond_the_static_array():
    """Host-side: a call whose pooled queries exceed 16 MiB is refused with
    FP2_EUNSUPPORTED and a message, before any device call (runs without a
    GPU); invalid parameters give the regular entry point's status."""
    fp2_mod.load()
    p = fp2_mod.make_params(32, 8, 128, 128, tau=1.0)
    S = 131072
    assert fp2_mod.fp2_select_workspace_size(p, 4, S, S) == SCRATCH_BYTES
    assert fp2_mod.fp2_select_workspace_size(p, 5, S, S) > SCRATCH_BYTES
    st = fp2_mod.fp2_select_blocks_noalloc(p, 5, S, S, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == fp2_mod.FP2_EUNSUPPORTED
    assert "scratch" in fp2_mod.last_error()
    bad = fp2_mod.make_params(32, 8, 96, 128, tau=1.0)
    assert fp2_mod.fp2_select_blocks_noalloc(bad, 1, 1024, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             None) == fp2_mod.FP2_EUNSUPPORTED
    p.tau = float("nan")
    assert fp2_mod.fp2_select_blocks_noalloc(p, 1, 1024, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             None) == fp2_mod.FP2_EINVAL
