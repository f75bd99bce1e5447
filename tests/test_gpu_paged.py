"""GPU parity of the paged-KV / continuous-batch path (chunked prefill over a
cached prefix, permuted 64-token pages with NaN canary pages)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import assert_mask_matches, check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


# page sizes on both copy paths: pages that fill whole 1 KB LDS copy ops
# (at least 32 rows for d = 128 in bf16, 64 for d = 64) take the per-tile
# offset table, smaller ones the per-copy cursor
@pytest.mark.parametrize("d,b,page", [(128, 128, 64), (128, 128, 16), (128, 128, 32), (128, 128, 128), (64, 64, 16),
                                      (64, 64, 64)])
def test_paged_matches_oracle_and_contiguous(gpu, d, b, page):
    hq, hkv = 8, 2
    kv_lens = [700, 1500, 2048, 333]
    q_lens = [700, 300, 1024, 333]
    print(f"[case] paged kv_lens={kv_lens} q_lens={q_lens} hq={hq} hkv={hkv} d={d} b={b} page={page}", flush=True)
    pb = synth.make_paged(11, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau)
    q = pb.q.cuda()
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, q, pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s, seq in enumerate(pb.seqs):
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        print(f"[paged] seq {s}: nqb={geo.nqb} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
        check_blocks(f64(out[cu[s]:cu[s + 1]]), O, geo, hkv, lse=f64(lse[cu[s]:cu[s + 1]]).T, L=L,
                     label=f"paged seq {s}")
        # the contiguous path on the same data gives bit-identical rows
        qc, kc, vc = seq["q"].cuda(), seq["k"].cuda(), seq["v"].cuda()
        i2, c2, pk2, pv2 = gpu.select_blocks(p, qc, kc, vc)
        o2 = gpu.sparse_prefill(p, qc, kc, vc, i2, c2, pk2, pv2)
        torch.cuda.synchronize()
        assert torch.equal(c2[0], cnt[s, :, :geo.nqb])
        assert torch.equal(o2, out[cu[s]:cu[s + 1]])


@pytest.mark.parametrize("page", [64, 16])
def test_paged_sequences_without_new_rows(gpu, page):
    """Continuous-batch slots with cached tokens but no new rows (q_len 0, in
    the middle and at the end of the batch): they get no output rows and no
    tiles.  The other sequences match the oracle and equal, bit for bit, the
    same call with the empty slots left out (each tile computes the same
    values whatever else the launch holds)."""
    hq, hkv, d, b = 8, 2, 128, 128
    kv_lens = [1500, 900, 1024, 64]
    q_lens = [700, 0, 300, 0]
    print(f"[case] paged empty slots kv_lens={kv_lens} q_lens={q_lens} page={page}", flush=True)
    pb = synth.make_paged(13, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau)
    q, kc, vc = pb.q.cuda(), pb.k_cache.cuda(), pb.v_cache.cuda()
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, q, pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), kc, vc,
        pb.page_table.cuda(), export_mask=True, return_lse=True)
    keep = [s for s in range(len(q_lens)) if q_lens[s] > 0]
    cu2 = torch.tensor(np.concatenate([[0], np.cumsum([q_lens[s] for s in keep])]), dtype=torch.int32)
    sk2 = torch.tensor([kv_lens[s] for s in keep], dtype=torch.int32)
    out2, lse2 = gpu.sparse_prefill_paged(p, q, cu2.cuda(), sk2.cuda(), max(q_lens), max(kv_lens), kc, vc,
                                          pb.page_table[keep].contiguous().cuda(), return_lse=True)
    torch.cuda.synchronize()
    assert out.shape[0] == sum(q_lens)
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    cu = pb.cu_seqlens_q.numpy()
    for s in keep:
        seq = pb.seqs[s]
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        check_blocks(f64(out[cu[s]:cu[s + 1]]), O, geo, hkv, lse=f64(lse[cu[s]:cu[s + 1]]).T, L=L,
                     label=f"paged empty slots seq {s}")


def test_paged_mixed_prefill_and_decode_rows(gpu):
    """One call mixing decode rows (a one-row new chunk after a cached prefix),
    a chunked prefill and a full prefill, as continuous batching issues them:
    a decode row is a query block of one row, selected and attended like any
    other.  Positions cover a decode row that opens a new key block (kv_len
    = 1025: its diagonal block holds the one new key) and one deep in a block."""
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens = [1500, 1025, 2048, 300, 4000]
    q_lens = [1, 1, 700, 300, 1]
    print(f"[case] mixed decode kv_lens={kv_lens} q_lens={q_lens}", flush=True)
    pb = synth.make_paged(13, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau)
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s, seq in enumerate(pb.seqs):
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        print(f"[mixed] seq {s}: q_len={q_lens[s]} nqb={geo.nqb} kept={int(kept_gpu.sum())}", flush=True)
        check_blocks(f64(out[cu[s]:cu[s + 1]]), O, geo, hkv, lse=f64(lse[cu[s]:cu[s + 1]]).T, L=L,
                     label=f"mixed seq {s}")


def _same_masks(m1, m2, lo, hi, b):
    """Exported masks of two calls agree on every defined entry (each
    sequence's query blocks; the lists up to their counts)."""
    for s in range(len(hi)):
        geo = A.geometry(hi[s] - lo[s], hi[s], b)
        c1, c2 = m1[1][s, :, :geo.nqb], m2[1][s, :, :geo.nqb]
        assert torch.equal(c1, c2), s
        k1 = kept_from_lists(m1[0][s, :, :geo.nqb], c1, geo.nkb)
        k2 = kept_from_lists(m2[0][s, :, :geo.nqb], c2, geo.nkb)
        assert np.array_equal(k1, k2), s


def _chunk_vs_oracle(seq, lo, hi, hkv, b, tau, mode, corr, o, lse, idx, cnt, label):
    """The rows [lo, hi) of one sequence (a chunk over the cached prefix
    [0, lo)) against the oracle: mask bit-exact outside the band, outputs and
    LSE per (query block, KV head) under the exported mask."""
    qn, kn, vn = f64(seq["q"][lo:hi]), f64(seq["k"][:hi]), f64(seq["v"][:hi])
    d = qn.shape[2]
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, mean_correction=corr, q_blocks=[], select_mode=mode)
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[:, :geo.nqb], cnt[:, :geo.nqb], geo.nkb)
    band = (A.union_band_mask(ref["S"], ref["thr"], hkv) if mode == "union"
            else A.score_band_mask(ref["S"], ref["thr"]))
    assert not ((kept_gpu != ref["kept"]) & ~band).any(), label
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), corr)
    check_blocks(f64(o), O, geo, hkv, lse=f64(lse).T, L=L, label=label)
    return ref


@pytest.mark.parametrize("mode", ["mean", "union", "max"])
def test_paged_block_sum_cache_chunked_prefill(gpu, mode):
    """Chunked prefill with the key-block sum cache (fp2_sparse_prefill_paged_
    pooled): each chunk's call reads the sums of the full blocks its earlier
    chunks wrote and must give bit-identical masks, outputs and LSE to the
    uncached call; the cache entries must be the row sums of the blocks."""
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    L = [2048, 1500]
    bounds = [[0, 700, 1300, 2048], [0, 500, 1000, 1500]]   # chunk ends, not block aligned
    print(f"[case] block-sum cache L={L} chunks={bounds} select={mode}", flush=True)
    pb = synth.make_paged(14, L, L, hq, hkv, d, b, page_size=page)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode=mode)
    kc, vc, tab = pb.k_cache.cuda(), pb.v_cache.cuda(), pb.page_table.cuda()
    bsk, bsv = gpu.block_sum_cache(p, kc)
    cached = torch.zeros(2, dtype=torch.int32, device="cuda")
    for c in range(3):
        lo = [bounds[s][c] for s in range(2)]
        hi = [bounds[s][c + 1] for s in range(2)]
        q = torch.cat([pb.seqs[s]["q"][lo[s]:hi[s]] for s in range(2)], 0).cuda()
        cu = torch.tensor([0, hi[0] - lo[0], hi[0] - lo[0] + hi[1] - lo[1]], dtype=torch.int32, device="cuda")
        sk = torch.tensor(hi, dtype=torch.int32, device="cuda")
        args = (p, q, cu, sk, max(h - l for h, l in zip(hi, lo)), max(hi), kc, vc, tab)
        o1, m1, l1 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
        o2, m2, l2 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True, pool_cache=(bsk, bsv, cached))
        torch.cuda.synchronize()
        # the cached call against the oracle, chunk by chunk
        off = 0
        for s in range(2):
            n = hi[s] - lo[s]
            _chunk_vs_oracle(pb.seqs[s], lo[s], hi[s], hkv, b, tau, mode, True, o2[off:off + n],
                             l2[off:off + n], m2[0][s], m2[1][s], f"cached chunk {c} seq {s}")
            off += n
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"chunk {c}"
        _same_masks(m1, m2, lo, hi, b)
        cached = (sk // b).to(torch.int32)
        # the cache now holds every full block of the prefix: the oracle's
        # block means times the block's key count
        for s in range(2):
            _, kbar, vbar, n_k = A.pool(f64(pb.seqs[s]["q"][:hi[s]]), f64(pb.seqs[s]["k"][:hi[s]]),
                                        f64(pb.seqs[s]["v"][:hi[s]]), hkv, b)
            for j in range(hi[s] // b):
                assert n_k[j] == b
                pg = int(pb.page_table[s, (j * b) // page])
                ksum, vsum = kbar[:, j] * n_k[j], vbar[:, j] * n_k[j]      # [Hkv, d]
                gk = bsk[pg].double().cpu().numpy()
                gv = bsv[pg].double().cpu().numpy()
                assert np.abs(gk - ksum).max() <= 1e-5 * np.abs(ksum).max() + 1e-4, (c, s, j)
                assert np.abs(gv - vsum).max() <= 1e-5 * np.abs(vsum).max() + 1e-4, (c, s, j)
        print(f"[cache] chunk {c}: q rows {hi[0] - lo[0]}+{hi[1] - lo[1]}, cached blocks now {cached.tolist()}",
              flush=True)
    # a repeat of the last chunk reads every full block from the cache
    o3, m3, l3 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True, pool_cache=(bsk, bsv, cached))
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    _same_masks(m1, m3, lo, hi, b)


def test_paged_block_sum_cache_without_correction(gpu):
    """The cached call with the mean correction off and NO value-sum cache
    (block_sums_v = NULL, which the header allows then): the V means are
    neither pooled nor cached, and each chunk's masks, outputs and LSE match
    the oracle without correction, and the uncached call bit for bit."""
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    L = [2048, 1500]
    bounds = [[0, 700, 1300, 2048], [0, 500, 1000, 1500]]
    print(f"[case] block-sum cache without correction, NULL V sums, L={L} chunks={bounds}", flush=True)
    pb = synth.make_paged(15, L, L, hq, hkv, d, b, page_size=page)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau, mean_correction=False)
    kc, vc, tab = pb.k_cache.cuda(), pb.v_cache.cuda(), pb.page_table.cuda()
    bsk, _ = gpu.block_sum_cache(p, kc)
    cached = torch.zeros(2, dtype=torch.int32, device="cuda")
    for c in range(3):
        lo = [bounds[s][c] for s in range(2)]
        hi = [bounds[s][c + 1] for s in range(2)]
        q = torch.cat([pb.seqs[s]["q"][lo[s]:hi[s]] for s in range(2)], 0).cuda()
        cu = torch.tensor([0, hi[0] - lo[0], hi[0] - lo[0] + hi[1] - lo[1]], dtype=torch.int32, device="cuda")
        sk = torch.tensor(hi, dtype=torch.int32, device="cuda")
        args = (p, q, cu, sk, max(h - l for h, l in zip(hi, lo)), max(hi), kc, vc, tab)
        o1, m1, l1 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
        o2, m2, l2 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True, pool_cache=(bsk, None, cached))
        torch.cuda.synchronize()
        off = 0
        for s in range(2):
            n = hi[s] - lo[s]
            _chunk_vs_oracle(pb.seqs[s], lo[s], hi[s], hkv, b, tau, "mean", False, o2[off:off + n], l2[off:off + n],
                             m2[0][s], m2[1][s], f"no-correction cached chunk {c} seq {s}")
            off += n
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"chunk {c}"
        _same_masks(m1, m2, lo, hi, b)
        cached = (sk // b).to(torch.int32)


@pytest.mark.parametrize("bad", ["past_end", "negative"])
def test_validate_rejects_bad_page_id_before_any_kernel(gpu, monkeypatch, bad):
    """FP2_VALIDATE=1: the paged call copies the lengths and the page table to
    the host and rejects a page id outside [0, num_pages) with FP2_EINVAL
    before anything is enqueued (the output buffer keeps its sentinel).  The
    same call on the valid table passes validation and equals the call
    without it.  (The invalid table is only ever passed with validation on.)"""
    monkeypatch.setenv("FP2_VALIDATE", "1")
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens, q_lens = [700, 1500], [700, 300]
    print(f"[case] FP2_VALIDATE bad page id ({bad}) kv_lens={kv_lens}", flush=True)
    pb = synth.make_paged(16, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    q, cu, sk = pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda()
    kc, vc = pb.k_cache.cuda(), pb.v_cache.cuda()
    tab_ok = pb.page_table.cuda()
    ref = gpu.sparse_prefill_paged(p, q, cu, sk, max(q_lens), max(kv_lens), kc, vc, tab_ok)
    torch.cuda.synchronize()
    n, msq, msk = len(kv_lens), max(q_lens), max(kv_lens)
    ws = torch.empty(gpu.fp2_paged_workspace_size(p, n, msq, msk), dtype=torch.uint8, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream

    def call(tab, out):
        return gpu.fp2_sparse_prefill_paged(p, n, q.data_ptr(), cu.data_ptr(), sk.data_ptr(), msq, msk, kc.data_ptr(),
                                            vc.data_ptr(), kc.shape[0], kc.shape[1], tab.data_ptr(), tab.shape[1],
                                            out.data_ptr(), None, None, None, ws.data_ptr(), ws.numel(), sh)

    # valid table under validation: same result as without it
    out = torch.full_like(ref, 7.0)
    assert call(tab_ok, out) == gpu.FP2_OK, gpu.last_error()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # one page id of sequence 1 (inside its seqlens_k) out of range
    tab = pb.page_table.clone()
    tab[1, 10] = kc.shape[0] if bad == "past_end" else -3
    tab_bad = tab.cuda()
    out = torch.full_like(ref, 7.0)
    st = call(tab_bad, out)
    msg = gpu.last_error()
    torch.cuda.synchronize()
    print(f"[validate] status {gpu.status_string(st)}: {msg}", flush=True)
    assert st == gpu.FP2_EINVAL and "page id" in msg
    assert bool((out == 7.0).all()), "a kernel ran after the validation error"


def _cache_chunking(seed):
    r = np.random.default_rng(9000 + seed)
    d = int(r.choice([64, 128]))
    b = int(r.choice([64, 128]))
    page = int(r.choice([p for p in (16, 32, 64, 128) if p <= b and b // p <= 64]))
    hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 4, 8]))
    n = int(r.integers(1, 4))
    lens = [int(r.integers(1500, 9000)) for _ in range(n)]
    nch = int(r.integers(2, 6))
    bounds = []
    for Ls in lens:
        cut = sorted(set(int(x) for x in r.integers(1, Ls, size=nch - 1)))
        if r.random() < 0.3:   # block-aligned cuts
            cut = sorted(set(max(b, (x // b) * b) for x in cut))
        bounds.append([0] + [x for x in cut if 0 < x < Ls] + [Ls])
    return dict(d=d, b=b, page=page, hkv=hkv, hq=G * hkv, lens=lens, bounds=bounds, tau=float(r.uniform(0.9, 2.0)),
                fp8=bool(r.random() < 0.3), mode=str(r.choice(["mean", "union", "max"])), corr=bool(r.random() < 0.8))


@pytest.mark.parametrize("seed", [5, 8, 10, 16])
def test_block_sum_cache_random_chunkings(gpu, seed):
    """Seeded chunked prefills of 1-3 sequences in 2-5 chunks (cuts at random
    or on block boundaries), bf16 or fp8, any selection rule: in every chunk
    the cached call equals the uncached one bit for bit (outputs, LSE and the
    defined mask entries), and each sequence's first and last query block of
    the chunk match the oracle."""
    c = _cache_chunking(seed)
    print(f"[case] block-sum cache random chunking seed={seed} {c}", flush=True)
    pb = synth.make_paged(500 + seed, c["lens"], c["lens"], c["hq"], c["hkv"], c["d"], c["b"], page_size=c["page"],
                          fp8=c["fp8"])
    scales = dict(fp8=True, q_scale=pb.q_scale.cuda(), k_scale=pb.k_scale.cuda(), v_scale=pb.v_scale.cuda()) \
        if c["fp8"] else {}
    p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], mean_correction=c["corr"],
                        select_mode=c["mode"], **scales)
    kc, vc, tab = pb.k_cache.cuda(), pb.v_cache.cuda(), pb.page_table.cuda()
    bsk, bsv = gpu.block_sum_cache(p, kc)
    n = len(c["lens"])
    cached = torch.zeros(n, dtype=torch.int32, device="cuda")
    for ck in range(max(len(bd) - 1 for bd in c["bounds"])):
        act = [s for s in range(n) if ck + 1 < len(c["bounds"][s])]
        lo = {s: c["bounds"][s][ck] for s in act}
        hi = {s: c["bounds"][s][ck + 1] for s in act}
        q = torch.cat([(pb.seqs[s]["qc"] if c["fp8"] else pb.seqs[s]["q"])[lo[s]:hi[s]] for s in act], 0).cuda()
        cu = [0]
        for s in act:
            cu.append(cu[-1] + hi[s] - lo[s])
        args = (p, q, torch.tensor(cu, dtype=torch.int32, device="cuda"),
                torch.tensor([hi[s] for s in act], dtype=torch.int32, device="cuda"),
                max(hi[s] - lo[s] for s in act), max(hi[s] for s in act), kc, vc, tab[act].contiguous())
        o1, m1, l1 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
        o2, m2, l2 = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True,
                                              pool_cache=(bsk, bsv, cached[act].contiguous()))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"chunk {ck}"
        _same_masks(m1, m2, [lo[s] for s in act], [hi[s] for s in act], c["b"])
        for ai, s in enumerate(act):
            seq = pb.seqs[s]
            if c["fp8"]:
                qn = oracle.dequantize(seq["qc"][lo[s]:hi[s]].numpy(), pb.q_scale.numpy(), 1)
                kn = oracle.dequantize(seq["kc"][:hi[s]].numpy(), pb.k_scale.numpy(), 1)
                vn = oracle.dequantize(seq["vc"][:hi[s]].numpy(), pb.v_scale.numpy(), 1)
            else:
                qn, kn, vn = f64(seq["q"][lo[s]:hi[s]]), f64(seq["k"][:hi[s]]), f64(seq["v"][:hi[s]])
            ref = A.sparse_prefill(qn, kn, vn, c["hkv"], c["b"], c["tau"], mean_correction=c["corr"], q_blocks=[],
                                   select_mode=c["mode"])
            geo = ref["geo"]
            kept = kept_from_lists(m2[0][ai, :, :geo.nqb], m2[1][ai, :, :geo.nqb], geo.nkb)
            band = (A.union_band_mask(ref["S"], ref["thr"], c["hkv"]) if c["mode"] == "union"
                    else A.score_band_mask(ref["S"], ref["thr"]))
            assert not ((kept != ref["kept"]) & ~band).any(), f"chunk {ck} seq {s}"
            ids = geo.q_block_ids()
            blocks = sorted({int(ids[0]), int(ids[-1])})
            O, L = A.attend(qn, kn, vn, kept, ref["kbar"], ref["vbar"], ref["n_k"], c["hkv"], c["b"],
                            1 / math.sqrt(c["d"]), c["corr"], q_blocks=blocks)
            check_blocks(f64(o2[cu[ai]:cu[ai + 1]]), O, geo, c["hkv"], fp8=c["fp8"], blocks=blocks,
                         lse=f64(l2[cu[ai]:cu[ai + 1]]).T, L=L, label=f"cache chunk {ck} seq {s}")
        for s in act:
            cached[s] = hi[s] // c["b"]
