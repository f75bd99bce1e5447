"""GPU parity of the FP8 path (OCP e4m3 inputs with per-head scales) against
the float64 oracle run on the dequantized inputs, through the C ABI.  The
kernel's own rounding (P stored as e4m3 for the P V product) is what the fp8
output tolerance covers; the selection runs on dequantized values in both."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import FP8_LSE_ABS, FP8_REL_L2, assert_mask_matches, check_blocks, kept_from_lists, rel_l2

pytestmark = pytest.mark.gpu

# LSE bound of the fp8 path (FP8_LSE_ABS = 0.08): P is stored as e4m3 codes
# read as a log-linear approximation of 2^x (each within a factor exp(+-0.0728)
# of the exact value) and the row sums are taken over the stored P, so a row
# dominated by a single key can have its normaliser off by up to 0.0728 (its
# output is not affected: numerator and normaliser share the same stored P).


class Fp8Case:
    def __init__(self, kind, seed, S, hq, hkv, d, b, Sq=None):
        print(f"[case] fp8 {kind} seed={seed} Sk={S} Sq={Sq or S} hq={hq} hkv={hkv} d={d} b={b}", flush=True)
        pr = synth.make_problem(kind, seed, S, hq, hkv, d, b, seqlen_q=Sq)
        self.qc, self.qs = synth.quantize_e4m3(pr.q, 1)
        self.kc, self.ks = synth.quantize_e4m3(pr.k, 1)
        self.vc, self.vs = synth.quantize_e4m3(pr.v, 1)
        # oracle inputs: the exact dequantized values (decoded from the format)
        self.q = oracle.dequantize(self.qc.numpy(), self.qs.numpy(), 1)
        self.k = oracle.dequantize(self.kc.numpy(), self.ks.numpy(), 1)
        self.v = oracle.dequantize(self.vc.numpy(), self.vs.numpy(), 1)
        self.dims = (hq, hkv, d, b)
        self.dev = [t.cuda() for t in (self.qc, self.kc, self.vc, self.qs, self.ks, self.vs)]

    def params(self, fp2, tau=float("inf"), **kw):
        hq, hkv, d, b = self.dims
        _, _, _, qs, ks, vs = self.dev
        return fp2.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs, k_scale=ks, v_scale=vs, **kw)


def _oracle_tau(q, k, v, hkv, b, target):
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


def _sparse_vs_oracle(fp2, c, target, tol=FP8_REL_L2):
    hq, hkv, d, b = c.dims
    tau = _oracle_tau(c.q, c.k, c.v, hkv, b, target)
    p = c.params(fp2, tau)
    qd, kd, vd = c.dev[:3]
    idx, cnt, pk, pv = fp2.select_blocks(p, qd, kd, vd)
    out, lse = fp2.sparse_prefill(p, qd, kd, vd, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(c.q, c.k, c.v, hkv, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
    assert np.abs(pk[0].double().cpu().numpy() - ref["kbar"]).max() < 2e-5
    O, L = A.attend(c.q, c.k, c.v, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    o = out.double().cpu().numpy().reshape(O.shape)
    print(f"[fp8 sparse] tau={tau:.3f} sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
    errs = check_blocks(o, O, geo, hkv, fp8=True, lse=lse[0].double().cpu().numpy(), L=L, label="fp8 sparse",
                        rel_tol=tol)
    return max(e["rel_l2"] for e in errs)


@pytest.mark.parametrize("S,Sq,target", [(4096, None, 0.8), (2500, None, 0.5), (4096, 1500, 0.7)])
def test_fp8_sparse_matches_oracle(gpu, S, Sq, target):
    _sparse_vs_oracle(gpu, Fp8Case("planted", 21, S, 8, 2, 128, 128, Sq), target)


@pytest.mark.parametrize("hq,hkv,d,b", [(8, 2, 128, 64), (8, 1, 64, 64), (4, 2, 64, 128), (16, 2, 128, 128)])
def test_fp8_other_shapes(gpu, hq, hkv, d, b):
    _sparse_vs_oracle(gpu, Fp8Case("planted", 22, 1500, hq, hkv, d, b), 0.5)


@pytest.mark.parametrize("S,Sq", [(2000, None), (3000, 777)])
def test_fp8_dense_matches_textbook(gpu, S, Sq):
    c = Fp8Case("planted", 23, S, 8, 2, 128, 128, Sq)
    p = c.params(gpu)
    qd, kd, vd = c.dev[:3]
    out, lse = gpu.dense_prefill(p, qd, kd, vd, return_lse=True)
    torch.cuda.synchronize()
    O, L = A.dense_attention(c.q, c.k, c.v, 2, 1 / math.sqrt(128))
    check_blocks(out.double().cpu().numpy(), O, A.geometry(O.shape[0], S, 128), 2, fp8=True,
                 lse=lse[0].double().cpu().numpy(), L=L, label="fp8 dense")


def test_fp8_tau_inf_sparse_equals_dense(gpu):
    c = Fp8Case("planted", 24, 1800, 8, 2, 128, 128)
    p = c.params(gpu)
    qd, kd, vd = c.dev[:3]
    idx, cnt, pk, pv = gpu.select_blocks(p, qd, kd, vd)
    out_s = gpu.sparse_prefill(p, qd, kd, vd, idx, cnt, pk, pv)
    out_d = gpu.dense_prefill(p, qd, kd, vd)
    torch.cuda.synchronize()
    assert (cnt[0].cpu().numpy() == np.arange(1, cnt.shape[2] + 1)[None, :]).all()
    assert torch.equal(out_s, out_d)


@pytest.mark.parametrize("shift", [200.0, 800.0, 8000.0])
@pytest.mark.parametrize("fp8", [True, False])
def test_large_logits_rerun(gpu, fp8, shift):
    """A block of keys whose logits exceed the sink block's by ~150, ~600 and
    ~6100 (log2 units): the first pass's reference (the sink chunk's maximum)
    is far below the row maximum, so the tile reruns with its reference at
    the largest exponent the first pass saw, which is exact for any finite
    logits; fp8 also exercises the per-superchunk P scaling over that range."""
    hq, hkv, d, b, S = 4, 1, 128, 128, 1024
    print(f"[case] large logits fp8={fp8} shift={shift}", flush=True)
    pr = synth.make_problem("iid", 25, S, hq, hkv, d, b)
    q = pr.q.float()
    k = pr.k.float()
    u = torch.ones(d) / math.sqrt(d)
    q += 6.0 * u                     # every query aligns with u
    k[600:700] += shift * u          # logits ~ 6 * shift / sqrt(d) nats above the rest
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    if fp8:
        qc, qs = synth.quantize_e4m3(q, 1)
        kc, ks = synth.quantize_e4m3(k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        qn = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
        kn = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
        vn = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
        p = gpu.make_params(hq, hkv, d, b, fp8=True, q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda())
        args = (qc.cuda(), kc.cuda(), vc.cuda())
        tol = FP8_REL_L2
    else:
        qn, kn, vn = (t.double().numpy() for t in (q, k, pr.v))
        p = gpu.make_params(hq, hkv, d, b)
        args = (q.cuda(), k.cuda(), pr.v.cuda())
        tol = 1e-2
    out, lse = gpu.dense_prefill(p, *args, return_lse=True)
    torch.cuda.synchronize()
    O, L = A.dense_attention(qn, kn, vn, hkv, 1 / math.sqrt(d))
    print(f"[rerun fp8={fp8} shift={shift}] lse range {L.min():.1f}..{L.max():.1f} nats "
          f"({(L.max() - L.min()) / math.log(2):.0f} log2 units)", flush=True)
    assert L.max() - L.min() > 0.3 * shift
    check_blocks(out.double().cpu().numpy(), O, A.geometry(S, S, b), hkv, fp8=fp8,
                 lse=lse[0].double().cpu().numpy(), L=L, label=f"rerun fp8={fp8} shift={shift}", rel_tol=tol)


# 64-row pages take the per-tile copy-offset table, 32-row pages (which do
# not fill whole 1 KB LDS copy ops in fp8) the per-copy cursor
@pytest.mark.parametrize("page", [64, 32])
def test_fp8_paged_matches_oracle_and_contiguous(gpu, page):
    hq, hkv, d, b = 8, 2, 128, 128
    kv_lens = [700, 1500, 2048, 333]
    q_lens = [700, 300, 1024, 333]
    print(f"[case] fp8 paged kv_lens={kv_lens} q_lens={q_lens}", flush=True)
    pb = synth.make_paged(12, kv_lens, q_lens, hq, hkv, d, b, page_size=page, fp8=True)
    qs, ks, vs = pb.q_scale.cuda(), pb.k_scale.cuda(), pb.v_scale.cuda()
    tau = 0.8
    p = gpu.make_params(hq, hkv, d, b, tau=tau, fp8=True, q_scale=qs, k_scale=ks, v_scale=vs)
    out, (idx, cnt) = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s, seq in enumerate(pb.seqs):
        qn = oracle.dequantize(seq["qc"].numpy(), pb.q_scale.numpy(), 1)
        kn = oracle.dequantize(seq["kc"].numpy(), pb.k_scale.numpy(), 1)
        vn = oracle.dequantize(seq["vc"].numpy(), pb.v_scale.numpy(), 1)
        ref = A.sparse_prefill(qn, kn, vn, hkv, b, tau, q_blocks=[])
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s, :, :geo.nqb], cnt[s, :, :geo.nqb], geo.nkb)
        assert_mask_matches(kept_gpu, ref["kept"], ref["S"], ref["thr"])
        O, _ = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
        check_blocks(out[cu[s]:cu[s + 1]].double().cpu().numpy(), O, geo, hkv, fp8=True, label=f"fp8 paged seq {s}")
        qc, kc, vc = seq["qc"].cuda(), seq["kc"].cuda(), seq["vc"].cuda()
        i2, c2, pk2, pv2 = gpu.select_blocks(p, qc, kc, vc)
        o2 = gpu.sparse_prefill(p, qc, kc, vc, i2, c2, pk2, pv2)
        torch.cuda.synchronize()
        assert torch.equal(c2[0], cnt[s, :, :geo.nqb])
        assert torch.equal(o2, out[cu[s]:cu[s + 1]])


def _code_steps(a, b):
    """Distance in e4m3 code steps between two uint8 code arrays (signed
    magnitude order; +0 and -0 are the same point)."""
    def ordinal(c):
        c = c.astype(np.int64)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return np.abs(ordinal(a) - ordinal(b))


@pytest.mark.parametrize("fp8_in,headroom", [(False, 1.25), (True, 1.25), (False, 0.5)])
def test_e4m3_output_codes(gpu, fp8_in, headroom):
    """e4m3 output (value = code * o_scale, RNE, saturated at 448) against
    the oracle's output encoded with the same scale, and against the same
    call's fp32 output encoded on the host.  headroom < 1 puts the largest
    outputs beyond 448 * o_scale (saturation)."""
    S, hq, hkv, d, b = 1536, 8, 2, 128, 128
    tau = 1.2
    if fp8_in:
        c = Fp8Case("planted", 21, S, hq, hkv, d, b)
        q, k, v = c.q, c.k, c.v
        qd, kd, vd = c.dev[:3]
        mk = lambda **kw: c.params(gpu, tau, **kw)  # noqa: E731
    else:
        print(f"[case] bf16 in, e4m3 out S={S} headroom={headroom}", flush=True)
        pr = synth.make_problem("planted", 21, S, hq, hkv, d, b)
        q, k, v = (t.double().numpy() for t in (pr.q, pr.k, pr.v))
        qd, kd, vd = pr.q.cuda(), pr.k.cuda(), pr.v.cuda()
        mk = lambda **kw: gpu.make_params(hq, hkv, d, b, tau=tau, **kw)  # noqa: E731
    p32 = mk(out_fp32=True)
    idx, cnt, pk, pv = gpu.select_blocks(p32, qd, kd, vd)
    out32 = gpu.sparse_prefill(p32, qd, kd, vd, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(q, k, v, hkv, b, tau, q_blocks=[])
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    O, _ = A.attend(q, k, v, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], hkv, b, 1 / math.sqrt(d), True)
    o_scale = float(np.abs(O).max()) / 448.0 * headroom
    os_dev = torch.tensor([o_scale], dtype=torch.float32, device="cuda")
    p8 = mk(out_fp8=True, o_scale=os_dev)
    codes = gpu.sparse_prefill(p8, qd, kd, vd, idx, cnt, pk, pv)
    torch.cuda.synchronize()
    assert codes.dtype == torch.uint8
    g = codes.cpu().numpy().reshape(O.shape)
    want = oracle.e4m3_encode(O / np.float64(np.float32(o_scale)))
    own = oracle.e4m3_encode(out32.double().cpu().numpy().reshape(O.shape) / np.float64(np.float32(o_scale)))
    st_ref, st_own = _code_steps(g, want), _code_steps(g, own)
    sat = float((np.abs(O) / o_scale > 448).mean())
    # decoded against the oracle's float64 output (values beyond the range
    # compare with their saturated value): e4m3 rounding (half a step, at
    # most 2^-4 relative, 2^-10 o_scale absolute in the subnormals) on top of
    # the attention path's own tolerance
    dec = oracle.e4m3_decode(g) * np.float64(np.float32(o_scale))
    Oc = np.clip(O, -448 * o_scale, 448 * o_scale)
    err = np.abs(dec - Oc)
    att_tol = FP8_REL_L2 if fp8_in else 2e-2
    bound = 2.0 ** -4 * np.abs(Oc) + 2.0 ** -10 * o_scale + att_tol * np.abs(Oc).max()
    e = rel_l2(dec, Oc)
    print(f"[e4m3 out fp8_in={fp8_in} headroom={headroom}] saturated={sat:.4f} rel_l2 vs oracle {e:.3e}, codes "
          f"equal to the oracle's {(st_ref == 0).mean():.4f}, to the encoded fp32 output {(st_own == 0).mean():.5f} "
          f"(max {st_own.max()} step)", flush=True)
    assert not np.any((g & 0x7F) == 0x7F), "an e4m3 NaN code was written"
    assert np.all(err <= bound) and e < FP8_REL_L2
    # per (query block, KV head): the attention tolerance plus e4m3 rounding
    # (relative error <= 2^-4 per element, so <= 2^-4 in rel-L2)
    check_blocks(dec, Oc, geo, hkv, fp8=True, label="e4m3 out", rel_tol=att_tol + 2.0 ** -4)
    assert st_own.max() <= 1 and (st_own == 0).mean() > 0.999
    if headroom < 1:
        assert sat > 0 and np.all((g[np.abs(O) / o_scale > 449] & 0x7F) == 0x7E)
