"""GPU edge cases of the contiguous path against the float64 oracle: the
sparsest mask the rule allows (tau = -inf keeps only the sink and diagonal
blocks, so every other visible block goes through the mean correction, over
several 128-pseudo-key rounds with a partial last one), single-row chunks
at the end of a long prefix, and the longest sequence the kernels accept."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


def _sample(geo, seed):
    rng = np.random.default_rng(seed)
    il = {0, 1, geo.nqb // 2, geo.nqb - 1, int(rng.integers(0, geo.nqb))}
    return sorted(geo.first_qblock + x for x in il if 0 <= x < geo.nqb)


# dropped blocks per row up to nkb - 2: 264 (b 64: four rounds of 64 pseudo-
# keys + 8) and 311 (b 128: two rounds of 128 + 55); the chunked case starts
# at block 273
@pytest.mark.parametrize("S,Sq,hq,hkv,d,b,fp8", [(17000, None, 4, 1, 64, 64, False),
                                                 (40000, None, 8, 2, 128, 128, False),
                                                 (40000, 5000, 8, 2, 128, 128, False),
                                                 (40000, None, 8, 2, 128, 128, True)])
def test_sink_and_diagonal_only(gpu, S, Sq, hq, hkv, d, b, fp8):
    pr = synth.make_problem("planted", 3, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] tau=-inf planted seed=3 Sk={S} Sq={Sq or S} hq={hq} hkv={hkv} d={d} b={b} fp8={fp8}", flush=True)
    tau = float("-inf")
    if fp8:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v, qs_, ks_, vs_ = (t.cuda() for t in (qc, kc, vc, qs, ks, vs))
        p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs_, k_scale=ks_, v_scale=vs_)
        # oracle inputs: the exact dequantized values (decoded from the format)
        qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
        kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
        vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        p = gpu.make_params(hq, hkv, d, b, tau=tau)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    geo = A.geometry(qn.shape[0], kn.shape[0], b)
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    # the mask is fixed by the rule alone: exactly blocks 0 and i
    want = np.zeros_like(kept_gpu)
    want[:, :, 0] = True
    want[:, np.arange(geo.nqb), geo.q_block_ids()] = True
    assert np.array_equal(kept_gpu, want)
    qbar, kbar, vbar, n_k = A.pool(qn, kn, vn, hkv, b)
    blocks = _sample(geo, 3)
    O, L = A.attend(qn, kn, vn, kept_gpu, kbar, vbar, n_k, hkv, b, 1 / math.sqrt(d), True, q_blocks=blocks)
    print(f"[edges] blocks={blocks} max dropped={geo.nkb - 2}", flush=True)
    check_blocks(f64(out), O, geo, hkv, fp8=fp8, blocks=blocks, lse=f64(lse[0]), L=L, label="sink+diagonal only")


# the smallest problems: a single key (the sink block is the diagonal block),
# one query row after a partial block, a partial first block, and five rows
# straddling the first block boundary (two query blocks, two key blocks)
@pytest.mark.parametrize("S,Sq,fp8", [(1, None, False), (100, 1, False), (37, None, False), (130, 5, False),
                                      (1, None, True), (130, 5, True)])
def test_smallest_problems(gpu, S, Sq, fp8):
    hq, hkv, d, b = 8, 2, 128, 128
    pr = synth.make_problem("planted", 4, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] smallest planted seed=4 Sk={S} Sq={Sq or S} fp8={fp8}", flush=True)
    tau = 0.5
    if fp8:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v, qs_, ks_, vs_ = (t.cuda() for t in (qc, kc, vc, qs, ks, vs))
        p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs_, k_scale=ks_, v_scale=vs_)
        qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
        kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
        vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        p = gpu.make_params(hq, hkv, d, b, tau=tau)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    dense, dlse = gpu.dense_prefill(p, q, k, v, return_lse=True)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    band = A.score_band_mask(ref["S"], ref["thr"])
    assert not ((kept_gpu != ref["kept"]) & ~band).any()
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    check_blocks(f64(out), O, geo, hkv, fp8=fp8, lse=f64(lse[0]), L=L, label=f"smallest Sk={S}")
    if geo.nkb == 1:
        # one key block: it is both sink and diagonal, nothing is dropped, and
        # the sparse call is the dense one bit for bit
        assert kept_gpu.all()
        assert torch.equal(out, dense) and torch.equal(lse, dlse)


@pytest.mark.parametrize("Sk", [5000, 5121, 5120])
def test_one_row_chunk_after_long_prefix(gpu, Sk):
    """A one-row chunk (decode-like row) at the end of a prefix, contiguous
    layout: a partial last block, a block opened by the row, a full block."""
    hq, hkv, d, b = 8, 2, 128, 128
    pr = synth.make_problem("planted", 4, Sk, hq, hkv, d, b, seqlen_q=1)
    print(f"[case] one-row chunk planted seed=4 Sk={Sk}", flush=True)
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau)
    geo = ref["geo"]
    assert geo.nqb == 1
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    band = A.score_band_mask(ref["S"], ref["thr"])
    assert not ((kept_gpu != ref["kept"]) & ~band).any()
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    print(f"[edges] one row Sk={Sk}: kept {int(kept_gpu.sum())} of {hkv * (geo.nkb)}", flush=True)
    check_blocks(f64(out), O, geo, hkv, lse=f64(lse[0]), L=L, label="one-row chunk")


@pytest.mark.slow
@pytest.mark.parametrize("d,b", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_longest_supported_sequence(gpu, d, b):
    """seqlen_k at fp2_max_seqlen_k (2.38M keys at d 128, b 128; 1.83M at
    d 128, b 64; 3.65M at d 64, b 128; 2.18M at d 64, b 64: the selection's
    score row and the correction's dropped-block list at their LDS limits,
    which differ per instance), a ragged 334-row chunk at its end; tau 1.0
    and -inf."""
    hq = hkv = 1
    Sk = gpu.fp2_max_seqlen_k(gpu.make_params(hq, hkv, d, b))
    Sq = 334
    pr = synth.make_problem("planted", 7, Sk, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] longest sequence planted seed=7 d={d} b={b} Sk={Sk} Sq={Sq}", flush=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    for tau in (1.0, float("-inf")):
        p = gpu.make_params(hq, hkv, d, b, tau=tau)
        idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
        out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
        torch.cuda.synchronize()
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
        band = A.score_band_mask(ref["S"], ref["thr"])
        assert not ((kept_gpu != ref["kept"]) & ~band).any()
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        print(f"[edges] Sk={Sk} tau={tau}: kept {int(kept_gpu.sum())} of {geo.nkb * geo.nqb} pairs", flush=True)
        check_blocks(f64(out), O, geo, hkv, lse=f64(lse[0]), L=L, label=f"longest tau={tau}")


@pytest.mark.parametrize("hq,hkv,fp8", [(64, 32, False), (128, 64, True)])
def test_most_heads(gpu, hq, hkv, fp8):
    """The largest head counts the pooling kernel takes at d 128 (a query
    row of all heads and a key row of K and V are 1024 16-byte tasks each):
    masks and outputs against the oracle."""
    d, b, S, tau = 128, 128, 1500, 0.8
    pr = synth.make_problem("planted", 9, S, hq, hkv, d, b)
    print(f"[case] most heads hq={hq} hkv={hkv} fp8={fp8} S={S}", flush=True)
    if fp8:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v, qs_, ks_, vs_ = (t.cuda() for t in (qc, kc, vc, qs, ks, vs))
        p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs_, k_scale=ks_, v_scale=vs_)
        qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
        kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
        vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        p = gpu.make_params(hq, hkv, d, b, tau=tau)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    band = A.score_band_mask(ref["S"], ref["thr"])
    assert not ((kept_gpu != ref["kept"]) & ~band).any()
    assert np.abs(f64(pk[0]) - ref["kbar"]).max() < 2e-5 and np.abs(f64(pv[0]) - ref["vbar"]).max() < 2e-5
    O, _ = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    print(f"[edges] hq={hq} hkv={hkv}: sparsity {A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
    check_blocks(f64(out), O, geo, hkv, fp8=fp8, label=f"most heads hq={hq}")
