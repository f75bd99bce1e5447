"""GPU parity of the contiguous path (select, sparse and dense attention)
against the float64 oracle, through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import assert_mask_matches, check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


def _case(kind, seed, S, hq, hkv, d, b, Sq=None):
    pr = synth.make_problem(kind, seed, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] {kind} seed={seed} Sk={S} Sq={Sq or S} hq={hq} hkv={hkv} d={d} b={b}", flush=True)
    return pr


def _oracle_tau(q, k, v, hkv, b, target):
    """tau giving ~target sparsity on the oracle's float64 scores."""
    qbar, kbar, vbar, n_k = A.pool(q, k, v, hkv, b)
    geo = A.geometry(q.shape[0], k.shape[0], b)
    S = A.block_scores(qbar, kbar, geo.q_block_ids())
    lo, hi = 0.0, 8.0
    for _ in range(50):
        mid = 0.5 * (lo + hi)
        kept, _ = A.select(S, geo.q_block_ids(), mid)
        if A.sparsity(kept, geo.q_block_ids()) > target:
            lo = mid
        else:
            hi = mid
    return hi


def _run_select(fp2, pr, hq, hkv, d, b, tau):
    p = fp2.make_params(hq, hkv, d, b, tau=tau)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    idx, cnt, pk, pv = fp2.select_blocks(p, q, k, v)
    torch.cuda.synchronize()
    return p, q, k, v, idx, cnt, pk, pv


@pytest.mark.parametrize("S,Sq,tau_target", [(2048, None, 0.6), (3000, None, 0.5), (3000, 1100, 0.5)])
def test_select_matches_oracle(gpu, S, Sq, tau_target):
    hq, hkv, d, b = 8, 2, 128, 128
    pr = _case("planted", 1, S, hq, hkv, d, b, Sq)
    q, k, v = f64(pr.q), f64(pr.k), f64(pr.v)
    tau = _oracle_tau(q, k, v, hkv, b, tau_target)
    p, *_, idx, cnt, pk, pv = _run_select(gpu, pr, hq, hkv, d, b, tau)
    ref = A.sparse_prefill(q, k, v, hkv, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    flips = assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
    assert flips <= max(2, kept_gpu.size // 1000)
    assert kept_gpu[:, :, 0].all()
    assert kept_gpu[:, np.arange(geo.nqb), geo.q_block_ids()].all()
    # pooled key / value blocks (fp32 accumulation of bf16 rows)
    assert np.abs(f64(pk[0]) - ref["kbar"]).max() < 2e-5
    assert np.abs(f64(pv[0]) - ref["vbar"]).max() < 2e-5
    sp = A.sparsity(kept_gpu, geo.q_block_ids())
    print(f"[select] tau={tau:.4f} sparsity={sp:.3f} band flips={flips}", flush=True)


def test_tiny_all_kept_fp32_out(gpu):
    """Tiny GQA prefill, 4 query heads per KV head, d 64, block 64, tau 2:
    every block is kept, output fp32; equals the oracle (and dense)."""
    hq, hkv, d, b, S = 4, 1, 64, 64, 1024
    pr = _case("iid", 0, S, hq, hkv, d, b)
    p = gpu.make_params(hq, hkv, d, b, tau=2.0, out_fp32=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, 2.0)
    kept_gpu = kept_from_lists(idx[0], cnt[0], ref["geo"].nkb)
    assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
    o = f64(out).reshape(ref["O"].shape)
    check_blocks(o, ref["O"], ref["geo"], hkv, lse=f64(lse[0]), L=ref["LSE"], label="tiny")
    assert np.abs(f64(lse[0]) - ref["LSE"]).max() < 1e-2


@pytest.mark.parametrize("S,Sq,target", [(4096, None, 0.7), (2500, None, 0.5), (4096, 1500, 0.6)])
def test_sparse_attention_matches_oracle(gpu, S, Sq, target):
    hq, hkv, d, b = 8, 2, 128, 128
    pr = _case("planted", 2, S, hq, hkv, d, b, Sq)
    qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    tau = _oracle_tau(qn, kn, vn, hkv, b, target)
    p, q, k, v, idx, cnt, pk, pv = _run_select(gpu, pr, hq, hkv, d, b, tau)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    geo = A.geometry(qn.shape[0], kn.shape[0], b)
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    qbar, kbar, vbar, n_k = A.pool(qn, kn, vn, hkv, b)
    O, L = A.attend(qn, kn, vn, kept_gpu, kbar, vbar, n_k, hkv, b, 1 / math.sqrt(d), True)
    print(f"[sparse] tau={tau:.3f} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
    check_blocks(f64(out), O, geo, hkv, lse=f64(lse[0]), L=L, label="sparse")


@pytest.mark.parametrize("S,Sq", [(2000, None), (3000, 777)])
def test_dense_matches_textbook(gpu, S, Sq):
    hq, hkv, d, b = 8, 2, 128, 128
    pr = _case("planted", 3, S, hq, hkv, d, b, Sq)
    p = gpu.make_params(hq, hkv, d, b)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    out, lse = gpu.dense_prefill(p, q, k, v, return_lse=True)
    torch.cuda.synchronize()
    O, L = A.dense_attention(f64(pr.q), f64(pr.k), f64(pr.v), hkv, 1 / math.sqrt(d))
    check_blocks(f64(out), O, A.geometry(O.shape[0], S, b), hkv, lse=f64(lse[0]), L=L, label="dense")


def test_tau_inf_sparse_equals_dense(gpu):
    hq, hkv, d, b, S = 8, 2, 128, 128, 1800
    pr = _case("planted", 4, S, hq, hkv, d, b)
    p, q, k, v, idx, cnt, pk, pv = _run_select(gpu, pr, hq, hkv, d, b, float("inf"))
    assert (cnt[0].cpu().numpy() == np.arange(1, cnt.shape[2] + 1)[None, :]).all()
    out_s = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    out_d = gpu.dense_prefill(p, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_d)


@pytest.mark.parametrize("batch,S,fp8", [(1, 40960, False), (2, 20480, False), (1, 81920, True)])
def test_tau_inf_sparse_equals_dense_head_groups(gpu, batch, S, fp8):
    """Dense launches whose K/V (all heads, over the batch) exceed 128 MiB take
    the KV heads two at a time; with every block kept, the sparse launch (all
    heads at once) must still give the same bits, output and LSE."""
    hq, hkv, d, b = 32, 8, 128, 128
    prs = [_case("iid", 20 + s, S, hq, hkv, d, b) for s in range(batch)]
    q, k, v = (torch.stack([getattr(p_, n) for p_ in prs]) for n in ("q", "k", "v"))
    extra = {}
    if fp8:
        q, qs = synth.quantize_e4m3(q[0], 1)
        k, ks = synth.quantize_e4m3(k[0], 1)
        v, vs = synth.quantize_e4m3(v[0], 1)
        q, k, v = q[None], k[None], v[None]
        extra = dict(fp8=True, q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda())
    assert 2 * batch * S * d * (1 if fp8 else 2) * hkv > 128 * 2**20
    p = gpu.make_params(hq, hkv, d, b, tau=float("inf"), **extra)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out_s, lse_s = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    out_d, lse_d = gpu.dense_prefill(p, q, k, v, return_lse=True)
    torch.cuda.synchronize()
    assert (cnt.cpu().numpy() == np.arange(1, cnt.shape[2] + 1)[None, None, :]).all()
    assert torch.equal(out_s, out_d) and torch.equal(lse_s, lse_d)
    assert torch.isfinite(out_d.float()).all()


def test_run_twice_bit_identical(gpu):
    hq, hkv, d, b, S = 8, 2, 128, 128, 2048
    pr = _case("planted", 5, S, hq, hkv, d, b)
    p, q, k, v, idx, cnt, pk, pv = _run_select(gpu, pr, hq, hkv, d, b, 1.0)
    o1 = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    idx2, cnt2, pk2, pv2 = gpu.select_blocks(p, q, k, v)
    o2 = gpu.sparse_prefill(p, q, k, v, idx2, cnt2, pk2, pv2)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2) and torch.equal(pk, pk2) and torch.equal(o1, o2)


def test_gqa_wider_group_and_small_blocks(gpu):
    """G = 8 (two workgroups per tile) and block 64 with head_dim 64."""
    for (hq, hkv, d, b) in [(16, 2, 128, 128), (8, 1, 64, 64)]:
        S = 1500
        pr = _case("planted", 6, S, hq, hkv, d, b)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
        tau = _oracle_tau(qn, kn, vn, hkv, b, 0.5)
        p, q, k, v, idx, cnt, pk, pv = _run_select(gpu, pr, hq, hkv, d, b, tau)
        out = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
        torch.cuda.synchronize()
        geo = A.geometry(S, S, b)
        kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
        qbar, kbar, vbar, n_k = A.pool(qn, kn, vn, hkv, b)
        O, _ = A.attend(qn, kn, vn, kept_gpu, kbar, vbar, n_k, hkv, b, 1 / math.sqrt(d), True)
        check_blocks(f64(out), O, geo, hkv, label=f"gqa hq={hq} hkv={hkv} d={d} b={b}")


@pytest.mark.parametrize("Sq", [None, 700])
def test_batch2_matches_per_sequence(gpu, Sq):
    hq, hkv, d, b, S = 8, 2, 128, 128, 1024
    prs = [_case("planted", 10 + s, S, hq, hkv, d, b, Sq) for s in range(2)]
    q = torch.stack([p.q for p in prs]).cuda()
    k = torch.stack([p.k for p in prs]).cuda()
    v = torch.stack([p.v for p in prs]).cuda()
    p = gpu.make_params(hq, hkv, d, b, tau=1.0)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    for s in range(2):
        i1, c1, k1, v1 = gpu.select_blocks(p, q[s], k[s], v[s])
        o1, l1 = gpu.sparse_prefill(p, q[s], k[s], v[s], i1, c1, k1, v1, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(c1[0], cnt[s]) and torch.equal(o1, out[s])
        assert torch.equal(l1[0], lse[s])   # [B, Hq, Sq] rows of sequence s
