"""GPU parity of the per-query-head block selections.  "union": every query
head of a GQA group applies the max-threshold rule to its own pooled query,
and the group keeps the union of its heads' blocks.  "max": the group's block
score is the largest of its heads' scores, thresholded once.  Checked against
the float64 oracle's select_union and select_head_max, on the contiguous and
the paged path, in bf16 and fp8."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


def _assert_mask(kept_gpu, ref, hkv, mode):
    """Bit-exact except within 1e-3 of a threshold: for "union" where some head
    of the group scores within 1e-3 of that head's threshold, for "max" where
    the group's score does.  Returns the number of such in-band flips."""
    band = A.union_band_mask(ref["S"], ref["thr"], hkv) if mode == "union" else A.score_band_mask(ref["S"], ref["thr"])
    diff = kept_gpu != ref["kept"]
    bad = diff & ~band
    assert not bad.any(), f"{int(bad.sum())} {mode}-mask entries differ outside the band, first at {np.argwhere(bad)[:5]}"
    return int((diff & band).sum())


MODES = ["union", "max"]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("S,Sq,hq,hkv,d,b,tau", [(3000, None, 8, 2, 128, 128, 0.6), (3000, 1100, 8, 2, 128, 128, 0.6),
                                                 (2500, None, 16, 2, 64, 64, 0.5), (4096, None, 4, 4, 128, 128, 0.8)])
def test_head_select_and_attention_match_oracle(gpu, S, Sq, hq, hkv, d, b, tau, mode):
    pr = synth.make_problem("planted", 5, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] {mode} planted seed=5 Sk={S} Sq={Sq or S} hq={hq} hkv={hkv} d={d} b={b} tau={tau}", flush=True)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode=mode)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode=mode)
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    flips = _assert_mask(kept_gpu, ref, hkv, mode)
    assert flips <= max(2, kept_gpu.size // 1000)
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    print(f"[{mode}] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} flips={flips}", flush=True)
    check_blocks(f64(out), O, geo, hkv, lse=f64(lse[0]), L=L, label=mode)


def test_head_select_with_one_head_per_group_equals_group_mean(gpu):
    """With G = 1 the three rules are the same computation: bit-identical masks."""
    hq = hkv = 4
    d = b = 128
    pr = synth.make_problem("planted", 6, 3000, hq, hkv, d, b)
    print("[case] union/max G=1 planted seed=6 Sk=3000", flush=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    res = []
    for mode in ("mean", "union", "max"):
        p = gpu.make_params(hq, hkv, d, b, tau=0.7, select_mode=mode)
        res.append(gpu.select_blocks(p, q, k, v))
    torch.cuda.synchronize()
    nkb = A.geometry(3000, 3000, b).nkb
    i0, c0, pk0, pv0 = res[0]
    for i1, c1, pk1, pv1 in res[1:]:
        assert torch.equal(c0, c1)
        assert np.array_equal(kept_from_lists(i0[0], c0[0], nkb), kept_from_lists(i1[0], c1[0], nkb))
        assert torch.equal(pk0, pk1) and torch.equal(pv0, pv1)


def test_head_max_differs_from_union_and_mean(gpu):
    """On i.i.d. inputs the heads of a group score differently and the three
    rules keep different blocks (the planted generator gives a group's heads
    one shared direction, and there they agree), so a kernel that took the
    union or the mean in the max mode fails here: the GPU's max mask must
    match the oracle's, and the oracle's max mask must differ from its union
    and mean masks outside the bands."""
    hq, hkv, d, b, S, tau = 8, 2, 128, 128, 4096, 0.1
    pr = synth.make_problem("iid", 5, S, hq, hkv, d, b)
    print(f"[case] max vs union vs mean iid seed=5 Sk={S} tau={tau}", flush=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode="max")
    idx, cnt, _, _ = gpu.select_blocks(p, q, k, v)
    torch.cuda.synchronize()
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    refs = {m: A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode=m) for m in ("max", "union", "mean")}
    geo = refs["max"]["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    _assert_mask(kept_gpu, refs["max"], hkv, "max")
    band = (A.score_band_mask(refs["max"]["S"], refs["max"]["thr"])
            | A.union_band_mask(refs["union"]["S"], refs["union"]["thr"], hkv)
            | A.score_band_mask(refs["mean"]["S"], refs["mean"]["thr"]))
    for other in ("union", "mean"):
        n = int(((refs["max"]["kept"] != refs[other]["kept"]) & ~band).sum())
        print(f"[max vs {other}] {n} blocks differ outside the bands", flush=True)
        assert n > 0


@pytest.mark.parametrize("mode", MODES)
def test_head_select_paged_matches_oracle_and_contiguous(gpu, mode):
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens = [700, 1500, 2048, 333]
    q_lens = [700, 300, 1024, 333]
    tau = 0.6
    print(f"[case] {mode} paged kv_lens={kv_lens} q_lens={q_lens} hq={hq} hkv={hkv} page={page}", flush=True)
    pb = synth.make_paged(12, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode=mode)
    q = pb.q.cuda()
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, q, pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s, seq in enumerate(pb.seqs):
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode=mode)
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        _assert_mask(kept_gpu, ref, hkv, mode)
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        print(f"[{mode} paged] seq {s}: nqb={geo.nqb} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}",
              flush=True)
        check_blocks(f64(out[cu[s]:cu[s + 1]]), O, geo, hkv, lse=f64(lse[cu[s]:cu[s + 1]]).T, L=L,
                     label=f"{mode} paged seq {s}")
        # the contiguous path on the same data: same masks, bit-identical rows
        qc, kc, vc = seq["q"].cuda(), seq["k"].cuda(), seq["v"].cuda()
        i2, c2, pk2, pv2 = gpu.select_blocks(p, qc, kc, vc)
        o2 = gpu.sparse_prefill(p, qc, kc, vc, i2, c2, pk2, pv2)
        torch.cuda.synchronize()
        assert torch.equal(c2[0], cnt[s, :, :geo.nqb])
        assert torch.equal(o2, out[cu[s]:cu[s + 1]])


@pytest.mark.parametrize("mode", MODES)
def test_head_select_fp8_matches_oracle(gpu, mode):
    """e4m3 inputs with per-head scales: the per-head pooled queries take the
    head's own q scale; masks and outputs against the oracle on the exactly
    dequantized values."""
    import oracle
    hq, hkv, d, b, S, tau = 8, 2, 128, 128, 3000, 0.6
    pr = synth.make_problem("planted", 8, S, hq, hkv, d, b)
    print(f"[case] {mode} fp8 planted seed=8 Sk={S} tau={tau}", flush=True)
    qc, qs = synth.quantize_e4m3(pr.q, 1)
    kc, ks = synth.quantize_e4m3(pr.k, 1)
    vc, vs = synth.quantize_e4m3(pr.v, 1)
    q, k, v, qs_, ks_, vs_ = (t.cuda() for t in (qc, kc, vc, qs, ks, vs))
    p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs_, k_scale=ks_, v_scale=vs_, select_mode=mode)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
    kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
    vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode=mode)
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    flips = _assert_mask(kept_gpu, ref, hkv, mode)
    O, _ = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    print(f"[{mode} fp8] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} flips={flips}", flush=True)
    check_blocks(f64(out), O, geo, hkv, fp8=True, label=f"{mode} fp8")
