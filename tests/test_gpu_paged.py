"""GPU parity of the paged-KV / continuous-batch path (chunked prefill over a
cached prefix, permuted 64-token pages with NaN canary pages)."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import (BF16_MAX_ABS, BF16_REL_L2, assert_mask_matches, f64, kept_from_lists, max_abs, rel_l2)

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
        o = f64(out[cu[s]:cu[s + 1]])
        e, m = rel_l2(o, O), max_abs(o, O)
        print(f"[paged] seq {s}: nqb={geo.nqb} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} "
              f"rel_l2={e:.2e} max_abs={m:.2e}", flush=True)
        assert e < BF16_REL_L2 and m < BF16_MAX_ABS
        assert np.abs(f64(lse[cu[s]:cu[s + 1]]).T - L).max() < 2e-2
        # the contiguous path on the same data gives bit-identical rows
        qc, kc, vc = seq["q"].cuda(), seq["k"].cuda(), seq["v"].cuda()
        i2, c2, pk2, pv2 = gpu.select_blocks(p, qc, kc, vc)
        o2 = gpu.sparse_prefill(p, qc, kc, vc, i2, c2, pk2, pv2)
        torch.cuda.synchronize()
        assert torch.equal(c2[0], cnt[s, :, :geo.nqb])
        assert torch.equal(o2, out[cu[s]:cu[s + 1]])


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
        o = f64(out[cu[s]:cu[s + 1]])
        e, m = rel_l2(o, O), max_abs(o, O)
        print(f"[mixed] seq {s}: q_len={q_lens[s]} nqb={geo.nqb} kept={int(kept_gpu.sum())} rel_l2={e:.2e} "
              f"max_abs={m:.2e}", flush=True)
        assert e < BF16_REL_L2 and m < BF16_MAX_ABS
        assert np.abs(f64(lse[cu[s]:cu[s + 1]]).T - L).max() < 2e-2


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


@pytest.mark.parametrize("mode", ["mean", "union"])
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
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"chunk {c}"
        _same_masks(m1, m2, lo, hi, b)
        cached = (sk // b).to(torch.int32)
        # the cache now holds every full block of the prefix: compare with the oracle's block sums
        for s in range(2):
            k = f64(pb.seqs[s]["k"][:hi[s]])
            v = f64(pb.seqs[s]["v"][:hi[s]])
            for j in range(hi[s] // b):
                pg = int(pb.page_table[s, (j * b) // page])
                ksum = k[j * b:(j + 1) * b].sum(0)          # [Hkv, d]
                vsum = v[j * b:(j + 1) * b].sum(0)
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
