"""GPU parity of the call options against the float64 oracle: the mean
correction switched off (dropped blocks leave the softmax entirely) and a
softmax scale other than 1/sqrt(d), in bf16 and fp8, contiguous and paged."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import assert_mask_matches, check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


def _inputs(pr, fp8):
    if not fp8:
        return [t.cuda() for t in (pr.q, pr.k, pr.v)], {}, (f64(pr.q), f64(pr.k), f64(pr.v))
    qc, qs = synth.quantize_e4m3(pr.q, 1)
    kc, ks = synth.quantize_e4m3(pr.k, 1)
    vc, vs = synth.quantize_e4m3(pr.v, 1)
    dev = [t.cuda() for t in (qc, kc, vc)]
    scales = dict(fp8=True, q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda())
    ref = tuple(oracle.dequantize(c.numpy(), s.numpy(), 1) for c, s in ((qc, qs), (kc, ks), (vc, vs)))
    return dev, scales, ref


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("corr,scale", [(False, 0.0), (True, 0.05), (False, 0.2)])
def test_correction_and_scale_options(gpu, fp8, corr, scale):
    hq, hkv, d, b, S, Sq, tau = 8, 2, 128, 128, 3000, 2200, 0.6
    pr = synth.make_problem("planted", 31, S, hq, hkv, d, b, seqlen_q=Sq)
    print(f"[case] options corr={corr} scale={scale} fp8={fp8} Sk={S} Sq={Sq}", flush=True)
    (q, k, v), scales, (qn, kn, vn) = _inputs(pr, fp8)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, softmax_scale=scale, mean_correction=corr, **scales)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    s = scale if scale > 0 else 1 / math.sqrt(d)
    ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, scale=s, mean_correction=corr, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, s, corr)
    print(f"[options] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
    check_blocks(f64(out), O, geo, hkv, fp8=fp8, lse=f64(lse[0]), L=L, label=f"options corr={corr} scale={scale}")


def test_paged_without_correction(gpu):
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens, q_lens = [1500, 2048, 700], [300, 2048, 700]
    tau = 0.6
    print(f"[case] paged without correction kv_lens={kv_lens} q_lens={q_lens}", flush=True)
    pb = synth.make_paged(32, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    p = gpu.make_params(hq, hkv, d, b, tau=tau, mean_correction=False)
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    cu = pb.cu_seqlens_q.numpy()
    for s_, seq in enumerate(pb.seqs):
        qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, mean_correction=False, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s_, :, :geo.nqb], cnt[s_, :, :geo.nqb], geo.nkb)
        assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
        O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), False)
        check_blocks(f64(out[cu[s_]:cu[s_ + 1]]), O, geo, hkv, lse=f64(lse[cu[s_]:cu[s_ + 1]]).T, L=L,
                     label=f"paged without correction seq {s_}")


def test_null_pooled_buffers(gpu):
    """pooled_v may be NULL for the selection (not written), and both pooled
    buffers may be NULL for attention without the correction: the same
    masks and outputs as with the buffers."""
    hq, hkv, d, b, S, tau = 8, 2, 128, 128, 2000, 0.6
    pr = synth.make_problem("planted", 33, S, hq, hkv, d, b)
    print("[case] NULL pooled buffers, S=2000", flush=True)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    p = gpu.make_params(hq, hkv, d, b, tau=tau, mean_correction=False)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    ref = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv)
    nqb, nkb = idx.shape[2], idx.shape[3]
    idx2 = torch.full_like(idx, -1)
    cnt2 = torch.empty_like(cnt)
    pk2 = torch.empty_like(pk)
    ws = torch.empty(gpu.fp2_select_workspace_size(p, 1, S, S), dtype=torch.uint8, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    st = gpu.fp2_select_blocks(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx2.data_ptr(), cnt2.data_ptr(),
                               pk2.data_ptr(), None, ws.data_ptr(), ws.numel(), sh)
    assert st == gpu.FP2_OK, gpu.last_error()
    out = torch.empty_like(ref)
    st = gpu.fp2_sparse_prefill(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx2.data_ptr(), cnt2.data_ptr(),
                                None, None, out.data_ptr(), None, sh)
    assert st == gpu.FP2_OK, gpu.last_error()
    torch.cuda.synchronize()
    assert torch.equal(cnt2, cnt) and torch.equal(pk2, pk)
    for h in range(hkv):
        for il in range(nqb):
            c = int(cnt[0, h, il])
            assert torch.equal(idx2[0, h, il, :c], idx[0, h, il, :c])
    assert torch.equal(out, ref)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("d,b", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_bf16_output_is_the_rounded_fp32_output(gpu, d, b, fp8):
    """The epilogue's output modes share one normalised value: the bf16
    output equals round-to-nearest-even of the fp32 output of the same call,
    bit for bit, in every kernel instance (and in both input precisions)."""
    hq, hkv, S, Sq = 8, 2, 2500, 1900
    print(f"[case] bf16 vs fp32 output d={d} b={b} fp8={fp8}", flush=True)
    pr = synth.make_problem("planted", 17, S, hq, hkv, d, b, seqlen_q=Sq)
    if fp8:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v = (t.cuda() for t in (qc, kc, vc))
        sc = dict(fp8=True, q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda())
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        sc = {}
    p16 = gpu.make_params(hq, hkv, d, b, tau=0.8, **sc)
    p32 = gpu.make_params(hq, hkv, d, b, tau=0.8, out_fp32=True, **sc)
    idx, cnt, pk, pv = gpu.select_blocks(p16, q, k, v)
    o16 = gpu.sparse_prefill(p16, q, k, v, idx, cnt, pk, pv)
    o32 = gpu.sparse_prefill(p32, q, k, v, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16 and o32.dtype == torch.float32
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_log_lines_and_unchanged_results(gpu, monkeypatch, capfd):
    """FP2_LOG=1: each entry point prints one line of its launch shape to
    stderr (select, sparse and dense attention, the paged call), and the
    results are the same bits as without it."""
    hq, hkv, d, b = 8, 2, 128, 128
    print("[case] FP2_LOG lines", flush=True)
    pr = synth.make_problem("planted", 18, 3000, hq, hkv, d, b)
    q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    pb = synth.make_paged(19, [1500, 2100], [700, 2100], hq, hkv, d, b, page_size=64)
    pargs = (p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), 2100, 2100, pb.k_cache.cuda(),
             pb.v_cache.cuda(), pb.page_table.cuda())

    def run():
        sel = gpu.select_blocks(p, q, k, v)
        o1 = gpu.sparse_prefill(p, q, k, v, *sel)
        o2 = gpu.dense_prefill(p, q, k, v)
        o3 = gpu.sparse_prefill_paged(*pargs)
        torch.cuda.synchronize()
        return o1, o2, o3

    monkeypatch.delenv("FP2_LOG", raising=False)
    ref = run()
    capfd.readouterr()
    monkeypatch.setenv("FP2_LOG", "1")
    got = run()
    err = capfd.readouterr().err
    monkeypatch.delenv("FP2_LOG")
    for a_, b_ in zip(ref, got):
        assert torch.equal(a_, b_)
    lines = [ln for ln in err.splitlines() if ln.startswith("[fp2] ")]
    assert any(ln.startswith("[fp2] select B=1 Sq=3000 Sk=3000 Hq=8 Hkv=2 d=128 b=128") for ln in lines), err
    assert any(ln.startswith("[fp2] sparse attention B=1 Sq=3000") for ln in lines), err
    assert any(ln.startswith("[fp2] dense attention B=1 Sq=3000") for ln in lines), err
    assert any(ln.startswith("[fp2] paged n=2 max_sq=2100 max_sk=2100 page=64") for ln in lines), err
