"""GPU parity of the per-query-head ("union") block selection: every query
head of a GQA group applies the max-threshold rule to its own pooled query,
and the group keeps the union of its heads' blocks.  Checked against the
float64 oracle's select_union, on the contiguous and the paged path."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from tests.helpers import BF16_MAX_ABS, BF16_REL_L2, FP8_REL_L2, f64, kept_from_lists, max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _assert_union_mask(kept_gpu, ref, hkv):
    """Bit-exact except where some head of the group scores within 1e-3 of
    that head's threshold; returns the number of such in-band flips."""
    band = A.union_band_mask(ref["S"], ref["thr"], hkv)
    diff = kept_gpu != ref["kept"]
    bad = diff & ~band
    assert not bad.any(), f"{int(bad.sum())} union-mask entries differ outside the band, first at {np.argwhere(bad)[:5]}"
    return int((diff & band).sum())


@pytest.mark.parametrize("S,Sq,hq,hkv,d,b,tau", [(3000, None, 8, 2, 128, 128, 0.6), (3000, 1100, 8, 2, 128, 128, 0.6),
                                                 (2500, None, 16, 2, 64, 64, 0.5), (4096, None, 4, 4, 128, 128, 0.8)])
def test_union_select_and_attention_match_oracle(gpu, S, Sq, hq, hkv, d, b, tau):
    pr = synth.make_problem("planted", 5, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] union planted seed=5 Sk={S} Sq={Sq or S} hq={hq} hkv={hkv} d={d} b={b} tau={tau}", flush=True)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode="union")
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode="union")
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    flips = _assert_union_mask(kept_gpu, ref, hkv)
    assert flips <= max(2, kept_gpu.size // 1000)
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    o = f64(out).reshape(O.shape)
    e, m = rel_l2(o, O), max_abs(o, O)
    print(f"[union] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} flips={flips} rel_l2={e:.2e} "
          f"max_abs={m:.2e}", flush=True)
    assert e < BF16_REL_L2 and m < BF16_MAX_ABS
    assert np.abs(f64(lse[0]) - L).max() < 2e-2


def test_union_with_one_head_per_group_equals_group_mean(gpu):
    """With G = 1 the two rules are the same computation: bit-identical masks."""
    hq = hkv = 4
    d = b = 128
    pr = synth.make_problem("planted", 6, 3000, hq, hkv, d, b)
    print("[case] union G=1 planted seed=6 Sk=3000", flush=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    res = []
    for mode in ("mean", "union"):
        p = gpu.make_params(hq, hkv, d, b, tau=0.7, select_mode=mode)
        res.append(gpu.select_blocks(p, q, k, v))
    torch.cuda.synchronize()
    (i0, c0, pk0, pv0), (i1, c1, pk1, pv1) = res
    assert torch.equal(c0, c1)
    nkb = A.geometry(3000, 3000, b).nkb
    assert np.array_equal(kept_from_lists(i0[0], c0[0], nkb), kept_from_lists(i1[0], c1[0], nkb))
    assert torch.equal(pk0, pk1) and torch.equal(pv0, pv1)


def test_union_paged_matches_oracle_and_contiguous(gpu):
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens = [700, 1500, 2048, 333]
    q_lens = [700, 300, 1024, 333]
    tau = 0.6
    print(f"[case] union paged kv_lens={kv_lens} q_lens={q_lens} hq={hq} hkv={hkv} page={page}", flush=True)
    pb = synth.make_paged(12, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, select_mode="union")
    q = pb.q.cuda()
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, q, pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s, seq in enumerate(pb.seqs):
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode="union")
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        _assert_union_mask(kept_gpu, ref, hkv)
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        o = f64(out[cu[s]:cu[s + 1]])
        e, m = rel_l2(o, O), max_abs(o, O)
        print(f"[union paged] seq {s}: nqb={geo.nqb} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} "
              f"rel_l2={e:.2e} max_abs={m:.2e}", flush=True)
        assert e < BF16_REL_L2 and m < BF16_MAX_ABS
        # the contiguous path on the same data: same masks, bit-identical rows
        qc, kc, vc = seq["q"].cuda(), seq["k"].cuda(), seq["v"].cuda()
        i2, c2, pk2, pv2 = gpu.select_blocks(p, qc, kc, vc)
        o2 = gpu.sparse_prefill(p, qc, kc, vc, i2, c2, pk2, pv2)
        torch.cuda.synchronize()
        assert torch.equal(c2[0], cnt[s, :, :geo.nqb])
        assert torch.equal(o2, out[cu[s]:cu[s + 1]])


def test_union_fp8_matches_oracle(gpu):
    """e4m3 inputs with per-head scales: the per-head pooled queries take the
    head's own q scale; masks and outputs against the oracle on the exactly
    dequantized values."""
    import oracle
    hq, hkv, d, b, S, tau = 8, 2, 128, 128, 3000, 0.6
    pr = synth.make_problem("planted", 8, S, hq, hkv, d, b)
    print(f"[case] union fp8 planted seed=8 Sk={S} tau={tau}", flush=True)
    qc, qs = synth.quantize_e4m3(pr.q, 1)
    kc, ks = synth.quantize_e4m3(pr.k, 1)
    vc, vs = synth.quantize_e4m3(pr.v, 1)
    q, k, v, qs_, ks_, vs_ = (t.cuda() for t in (qc, kc, vc, qs, ks, vs))
    p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs_, k_scale=ks_, v_scale=vs_, select_mode="union")
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
    kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
    vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[], select_mode="union")
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    flips = _assert_union_mask(kept_gpu, ref, hkv)
    O, _ = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    e = rel_l2(f64(out).reshape(O.shape), O)
    print(f"[union fp8] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f} flips={flips} rel_l2={e:.2e}", flush=True)
    assert e < FP8_REL_L2
