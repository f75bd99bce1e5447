"""Seeded random configurations against the float64 oracle: sequence and
chunk lengths, GQA ratio, head dim, block size, threshold, precision,
selection rule and correction drawn per case (a fixed list, the same on
every run), covering combinations the targeted tests do not; small cases
(up to 2.6K keys) checked whole, and large ones (4K-24K keys, more tiles
than compute units) on sampled query blocks."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attention as A
from tests.helpers import check_blocks, f64, kept_from_lists

pytestmark = pytest.mark.gpu


def _config(seed):
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([64, 128]))
    b = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 3]))
    G = int(r.choice([1, 2, 4, 8]))
    Sk = int(r.integers(b + 1, 2600))
    Sq = int(r.integers(1, Sk + 1)) if r.random() < 0.5 else Sk
    return dict(d=d, b=b, hkv=hkv, hq=G * hkv, Sk=Sk, Sq=Sq, tau=float(r.uniform(0.0, 2.5)),
                fp8=bool(r.random() < 0.35), mode=_mode(r.random()), corr=bool(r.random() < 0.8),
                kind=str(r.choice(["planted", "iid"])))


def _mode(u):
    """Selection rule from one uniform draw: 15% union, 15% head max, else group mean."""
    return "union" if u < 0.15 else "max" if u < 0.3 else "mean"


@pytest.mark.parametrize("seed", range(12))
def test_random_config(gpu, seed):
    c = _config(seed)
    print(f"[case] random seed={seed} {c}", flush=True)
    pr = synth.make_problem(c["kind"], 40 + seed, c["Sk"], c["hq"], c["hkv"], c["d"], c["b"], seqlen_q=c["Sq"])
    mode = c["mode"]
    if c["fp8"]:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v = (t.cuda() for t in (qc, kc, vc))
        p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], mean_correction=c["corr"], fp8=True,
                            q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda(), select_mode=mode)
        qn, kn, vn = (oracle.dequantize(x.numpy(), y.numpy(), 1) for x, y in ((qc, qs), (kc, ks), (vc, vs)))
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], mean_correction=c["corr"],
                            select_mode=mode)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(qn, kn, vn, c["hkv"], c["b"], c["tau"], mean_correction=c["corr"], q_blocks=[],
                           select_mode=mode)
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    band = A.union_band_mask(ref["S"], ref["thr"], c["hkv"]) if mode == "union" else A.score_band_mask(ref["S"], ref["thr"])
    assert not ((kept_gpu != ref["kept"]) & ~band).any()
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], c["hkv"], c["b"],
                    1 / math.sqrt(c["d"]), c["corr"])
    print(f"[random] sparsity={A.sparsity(kept_gpu, geo.q_block_ids()):.3f}", flush=True)
    check_blocks(f64(out), O, geo, c["hkv"], fp8=c["fp8"], lse=f64(lse[0]), L=L, label=f"random {seed}")


def _paged_config(seed):
    r = np.random.default_rng(2000 + seed)
    d = int(r.choice([64, 128]))
    b = int(r.choice([64, 128]))
    page = int(r.choice([p for p in (16, 32, 64, 128) if p <= b and b // p <= 64]))
    hkv = int(r.choice([1, 2]))
    G = int(r.choice([1, 4, 8]))
    n = int(r.integers(1, 5))
    kv = [int(r.integers(1, 2500)) for _ in range(n)]
    ql = [int(r.integers(1, L + 1)) if r.random() < 0.6 else L for L in kv]
    return dict(d=d, b=b, page=page, hkv=hkv, hq=G * hkv, kv=kv, q=ql, tau=float(r.uniform(0.2, 2.0)),
                fp8=bool(r.random() < 0.35), mode=_mode(r.random()))


@pytest.mark.parametrize("seed", range(6))
def test_random_paged_batch(gpu, seed):
    c = _paged_config(seed)
    print(f"[case] random paged seed={seed} {c}", flush=True)
    pb = synth.make_paged(60 + seed, c["kv"], c["q"], c["hq"], c["hkv"], c["d"], c["b"], page_size=c["page"],
                          fp8=c["fp8"])
    mode = c["mode"]
    scales = dict(fp8=True, q_scale=pb.q_scale.cuda(), k_scale=pb.k_scale.cuda(), v_scale=pb.v_scale.cuda()) \
        if c["fp8"] else {}
    p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], select_mode=mode, **scales)
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(c["q"]), max(c["kv"]), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s_, seq in enumerate(pb.seqs):
        if c["fp8"]:
            # oracle inputs: the exact dequantized values (decoded from the format)
            qn = oracle.dequantize(seq["qc"].numpy(), pb.q_scale.numpy(), 1)
            kn = oracle.dequantize(seq["kc"].numpy(), pb.k_scale.numpy(), 1)
            vn = oracle.dequantize(seq["vc"].numpy(), pb.v_scale.numpy(), 1)
        else:
            qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, c["hkv"], c["b"], c["tau"], q_blocks=[], select_mode=mode)
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s_, :, :geo.nqb], cnt[s_, :, :geo.nqb], geo.nkb)
        band = (A.union_band_mask(ref["S"], ref["thr"], c["hkv"]) if mode == "union"
                else A.score_band_mask(ref["S"], ref["thr"]))
        assert not ((kept_gpu != ref["kept"]) & ~band).any(), s_
        O, Lr = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], c["hkv"], c["b"],
                         1 / math.sqrt(c["d"]), True)
        check_blocks(f64(out[cu[s_]:cu[s_ + 1]]), O, geo, c["hkv"], fp8=c["fp8"],
                     lse=f64(lse[cu[s_]:cu[s_ + 1]]).T, L=Lr,
                     label=f"random paged {seed} seq {s_} Sk={c['kv'][s_]} Sq={c['q'][s_]}")


def _large_config(seed):
    r = np.random.default_rng(5000 + seed)
    d = int(r.choice([64, 128]))
    b = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    Sk = int(r.integers(4096, 24000))
    Sq = Sk if r.random() < 0.6 else int(r.integers(1, Sk + 1))
    c = dict(d=d, b=b, hkv=hkv, hq=G * hkv, Sk=Sk, Sq=Sq, tau=float(r.uniform(0.8, 2.2)),
             fp8=bool(r.random() < 0.3), mode=str(r.choice(["mean", "mean", "mean", "union", "max"])),
             corr=bool(r.random() < 0.85), kind=str(r.choice(["planted", "planted", "iid"])))
    if c["kind"] == "iid":
        c["tau"] *= 0.1     # i.i.d. block scores spread ~10x less than planted ones
    return c


# 502 to 5152 tiles per launch: more than the 256 compute units, so that the
# persistent workgroups take tiles from the tile-queue counters (the small
# configurations above stay below that)
@pytest.mark.parametrize("seed", [0, 2, 10, 12, 16, 21, 31, 39])
def test_random_large_config(gpu, seed):
    """Seeded configurations of 4K-24K keys: the whole block mask against the
    oracle, and the outputs and LSE of the first, the last and six seeded
    query blocks per KV head, each (query block, KV head) on its own."""
    c = _large_config(seed)
    print(f"[case] random large seed={seed} {c}", flush=True)
    pr = synth.make_problem(c["kind"], 900 + seed, c["Sk"], c["hq"], c["hkv"], c["d"], c["b"], seqlen_q=c["Sq"])
    mode = c["mode"]
    if c["fp8"]:
        qc, qs = synth.quantize_e4m3(pr.q, 1)
        kc, ks = synth.quantize_e4m3(pr.k, 1)
        vc, vs = synth.quantize_e4m3(pr.v, 1)
        q, k, v = (t.cuda() for t in (qc, kc, vc))
        p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], mean_correction=c["corr"], fp8=True,
                            q_scale=qs.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda(), select_mode=mode)
        qn, kn, vn = (oracle.dequantize(x.numpy(), y.numpy(), 1) for x, y in ((qc, qs), (kc, ks), (vc, vs)))
    else:
        q, k, v = (t.cuda() for t in (pr.q, pr.k, pr.v))
        p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], mean_correction=c["corr"],
                            select_mode=mode)
        qn, kn, vn = f64(pr.q), f64(pr.k), f64(pr.v)
    idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
    out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
    torch.cuda.synchronize()
    ref = A.sparse_prefill(qn, kn, vn, c["hkv"], c["b"], c["tau"], mean_correction=c["corr"], q_blocks=[],
                           select_mode=mode)
    geo = ref["geo"]
    kept_gpu = kept_from_lists(idx[0], cnt[0], geo.nkb)
    band = A.union_band_mask(ref["S"], ref["thr"], c["hkv"]) if mode == "union" else A.score_band_mask(ref["S"], ref["thr"])
    assert not ((kept_gpu != ref["kept"]) & ~band).any()
    ids = geo.q_block_ids()
    rng = np.random.default_rng(seed)
    blocks = sorted({int(ids[0]), int(ids[-1]), *(int(x) for x in rng.choice(ids, size=min(6, len(ids)), replace=False))})
    O, L = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], c["hkv"], c["b"],
                    1 / math.sqrt(c["d"]), c["corr"], q_blocks=blocks)
    print(f"[random large] sparsity={A.sparsity(kept_gpu, ids):.3f} blocks={blocks}", flush=True)
    check_blocks(f64(out), O, geo, c["hkv"], fp8=c["fp8"], blocks=blocks, lse=f64(lse[0]), L=L,
                 label=f"random large {seed}")


def _large_paged_config(seed):
    r = np.random.default_rng(7000 + seed)
    d = int(r.choice([64, 128]))
    b = int(r.choice([64, 128]))
    page = int(r.choice([p for p in (16, 32, 64, 128) if p <= b and b // p <= 64]))
    hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 4, 8]))
    n = int(r.integers(2, 6))
    kv = [int(r.integers(2000, 20000)) for _ in range(n)]
    ql = [int(r.integers(1, L + 1)) if r.random() < 0.5 else L for L in kv]
    return dict(d=d, b=b, page=page, hkv=hkv, hq=G * hkv, kv=kv, q=ql, tau=float(r.uniform(0.9, 2.0)),
                fp8=bool(r.random() < 0.3), mode=str(r.choice(["mean", "mean", "union", "max"])))


@pytest.mark.parametrize("seed", [0, 5, 12, 20])
def test_random_large_paged_batch(gpu, seed):
    """Seeded continuous batches of 2-5 sequences of 2K-20K keys (chunked
    prefills among them) over permuted pages of 16-128 tokens: each
    sequence's whole mask against the oracle, and the outputs and LSE of its
    first, last and three seeded query blocks per KV head."""
    c = _large_paged_config(seed)
    print(f"[case] random large paged seed={seed} {c}", flush=True)
    pb = synth.make_paged(300 + seed, c["kv"], c["q"], c["hq"], c["hkv"], c["d"], c["b"], page_size=c["page"],
                          fp8=c["fp8"])
    mode = c["mode"]
    scales = dict(fp8=True, q_scale=pb.q_scale.cuda(), k_scale=pb.k_scale.cuda(), v_scale=pb.v_scale.cuda()) \
        if c["fp8"] else {}
    p = gpu.make_params(c["hq"], c["hkv"], c["d"], c["b"], tau=c["tau"], select_mode=mode, **scales)
    out, (idx, cnt), lse = gpu.sparse_prefill_paged(
        p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(c["q"]), max(c["kv"]), pb.k_cache.cuda(),
        pb.v_cache.cuda(), pb.page_table.cuda(), export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "a canary (NaN) page was read"
    cu = pb.cu_seqlens_q.numpy()
    for s_, seq in enumerate(pb.seqs):
        if c["fp8"]:
            qn = oracle.dequantize(seq["qc"].numpy(), pb.q_scale.numpy(), 1)
            kn = oracle.dequantize(seq["kc"].numpy(), pb.k_scale.numpy(), 1)
            vn = oracle.dequantize(seq["vc"].numpy(), pb.v_scale.numpy(), 1)
        else:
            qn, kn, vn = f64(seq["q"]), f64(seq["k"]), f64(seq["v"])
        ref = A.sparse_prefill(qn, kn, vn, c["hkv"], c["b"], c["tau"], q_blocks=[], select_mode=mode)
        geo = ref["geo"]
        kept_gpu = kept_from_lists(idx[s_, :, :geo.nqb], cnt[s_, :, :geo.nqb], geo.nkb)
        band = (A.union_band_mask(ref["S"], ref["thr"], c["hkv"]) if mode == "union"
                else A.score_band_mask(ref["S"], ref["thr"]))
        assert not ((kept_gpu != ref["kept"]) & ~band).any(), s_
        ids = geo.q_block_ids()
        rng = np.random.default_rng(10 * seed + s_)
        blocks = sorted({int(ids[0]), int(ids[-1]),
                         *(int(x) for x in rng.choice(ids, size=min(3, len(ids)), replace=False))})
        O, Lr = A.attend(qn, kn, vn, kept_gpu, ref["kbar"], ref["vbar"], ref["n_k"], c["hkv"], c["b"],
                         1 / math.sqrt(c["d"]), True, q_blocks=blocks)
        check_blocks(f64(out[cu[s_]:cu[s_ + 1]]), O, geo, c["hkv"], fp8=c["fp8"], blocks=blocks,
                     lse=f64(lse[cu[s_]:cu[s_ + 1]]).T, L=Lr,
                     label=f"random large paged {seed} seq {s_} Sk={c['kv'][s_]} Sq={c['q'][s_]}")
