"""GPU parity at the full sizes of the benchmark workloads (32K and 128K
layers in bf16, the 128K layer in FP8 at the three sparsity levels the
benchmark times, the paged six-sequence batch), in the
launch configuration bench.py times: the whole layer runs on the GPU through
the C ABI; the float64 oracle then checks every KV group on its own (pool,
score and select over the whole sequence -> the group's full block mask;
attention under the GPU's mask of every query block at 32K and of 16 sampled
query blocks at 128K, the first and the last among them -> those rows of the
output and their LSE), each (query block, KV head) held to the tolerance on
its own."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import assert_mask_matches, check_blocks, kept_from_lists, tau_table

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

N_SAMPLED = 16   # query blocks per KV head checked at 128K


def _sample_blocks(nqb, first_qb, seed, n=N_SAMPLED):
    """n seeded query blocks of a sequence (local ids 0 .. nqb-1), always
    including the first and the last; all of them when nqb <= n."""
    if nqb <= n:
        return [first_qb + x for x in range(nqb)]
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, nqb - 1), size=n - 2, replace=False)
    return [first_qb + int(x) for x in sorted({0, nqb - 1, *mid.tolist()})]


def _check_group(h, G, q, k, v, tau, b, idx, cnt, out, lse, fp8, seed, label, all_blocks=False):
    """q [Sq, G, d], k/v [Sk, 1, d] float64 of KV group h; idx/cnt the GPU
    lists of that group; out [Sq, G, d] and lse [G, Sq] the GPU results."""
    ref = A.sparse_prefill(q, k, v, 1, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[None], cnt[None], geo.nkb)
    flips = assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
    blocks = (list(geo.q_block_ids()) if all_blocks else _sample_blocks(geo.nqb, geo.first_qblock, seed))
    d = q.shape[2]
    O, L = A.attend(q, k, v, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], 1, b, 1 / math.sqrt(d), True,
                    q_blocks=blocks)
    sp = A.sparsity(kept_gpu, geo.q_block_ids())
    print(f"[{label} h={h}] nqb={geo.nqb} sparsity={sp:.3f} band flips={flips} blocks checked={len(blocks)}",
          flush=True)
    check_blocks(out, O, geo, 1, fp8=fp8, blocks=blocks, lse=lse, L=L, label=f"{label} h={h}")
    return ref


@pytest.mark.parametrize("workload,fp8,sparsity", [("llama8b_s32k_bf16", False, 0.70),
                                                    ("llama8b_s128k_bf16", False, 0.80),
                                                    ("llama8b_s128k_fp8", True, 0.80),
                                                    ("llama8b_s128k_fp8", True, 0.85),
                                                    ("llama8b_s128k_fp8", True, 0.90)])
def test_fullsize_contiguous(gpu, workload, fp8, sparsity):
    w = synth.WORKLOADS[workload]
    S, hq, hkv, d, b = w["seqlen"], w["hq"], w["hkv"], w["d"], w["block"]
    tau = tau_table()[f"{workload}@{sparsity:.2f}"]["tau"]
    print(f"[case] {workload} S={S} tau={tau:.4f}", flush=True)
    prob = synth.make_problem(w["kind"], 0, S, hq, hkv, d, b)
    G = hq // hkv
    if fp8:
        qc, qs = synth.quantize_e4m3(prob.q, 1)
        kc, ks = synth.quantize_e4m3(prob.k, 1)
        vc, vs = synth.quantize_e4m3(prob.v, 1)
        dev = [t.cuda() for t in (qc, kc, vc, qs, ks, vs)]
        p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=dev[3], k_scale=dev[4], v_scale=dev[5])
    else:
        dev = [t.cuda() for t in (prob.q, prob.k, prob.v)]
        p = gpu.make_params(hq, hkv, d, b, tau=tau)
    qd, kd, vd = dev[:3]
    idx, cnt, pk, pv = gpu.select_blocks(p, qd, kd, vd)
    out, lse = gpu.sparse_prefill(p, qd, kd, vd, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    out_h = out.double().cpu().numpy()
    lse_h = lse[0].double().cpu().numpy()
    idx_h, cnt_h = idx[0].cpu(), cnt[0].cpu()
    pk_h = pk[0].double().cpu().numpy()
    del out, lse, idx, cnt, pk, pv, dev, qd, kd, vd
    torch.cuda.empty_cache()
    for h in range(hkv):
        sl = slice(h * G, (h + 1) * G)
        if fp8:
            q = oracle.dequantize(qc[:, sl].numpy(), qs[sl].numpy(), 1)
            k = oracle.dequantize(kc[:, h:h + 1].numpy(), ks[h:h + 1].numpy(), 1)
            v = oracle.dequantize(vc[:, h:h + 1].numpy(), vs[h:h + 1].numpy(), 1)
        else:
            q = prob.q[:, sl].double().numpy()
            k = prob.k[:, h:h + 1].double().numpy()
            v = prob.v[:, h:h + 1].double().numpy()
        ref = _check_group(h, G, q, k, v, tau, b, idx_h[h], cnt_h[h], out_h[:, sl], lse_h[sl], fp8, h,
                           f"{workload}@{sparsity:.2f}", all_blocks=S <= 32768)
        assert np.abs(pk_h[h] - ref["kbar"][0]).max() < 2e-5


def test_fullsize_paged_batch6(gpu):
    w = synth.WORKLOADS["paged_batch6"]
    hq, hkv, d, b = w["hq"], w["hkv"], w["d"], w["block"]
    tau = tau_table()["paged_batch6@0.80"]["tau"]
    kv_lens, q_lens = w["kv_lens"], w["q_lens"]
    print(f"[case] paged_batch6 kv={kv_lens} q={q_lens} tau={tau:.4f}", flush=True)
    pb = synth.make_paged(0, kv_lens, q_lens, hq, hkv, d, b, page_size=w["page_size"])
    p = gpu.make_params(hq, hkv, d, b, tau=tau)
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    out_h = out.double().cpu().numpy()
    lse_h = lse.double().cpu().numpy()
    idx_h, cnt_h = idx.cpu(), cnt.cpu()
    cu = pb.cu_seqlens_q.numpy()
    G = hq // hkv
    for s, seq in enumerate(pb.seqs):
        for h in range(hkv):
            sl = slice(h * G, (h + 1) * G)
            q = seq["q"][:, sl].double().numpy()
            k = seq["k"][:, h:h + 1].double().numpy()
            v = seq["v"][:, h:h + 1].double().numpy()
            nqb = A.geometry(q.shape[0], k.shape[0], b).nqb
            _check_group(h, G, q, k, v, tau, b, idx_h[s, h, :nqb], cnt_h[s, h, :nqb], out_h[cu[s]:cu[s + 1], sl],
                         lse_h[cu[s]:cu[s + 1], sl].T, False, 100 * s + h, f"paged_batch6 seq {s}")
