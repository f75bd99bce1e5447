"""Benchmark of the block-sparse prefill hot path on one MI355X.

A step = one block-sparse causal prefill of one attention layer on the 128K
workload (batch 1, 32 query / 8 KV heads, head_dim 128, block 128, planted
retrieval structure + RoPE, tau for ~80% block sparsity): fp2_select_blocks
(pool + score + select) followed by fp2_sparse_prefill (attention with mean
correction).  The in-house dense causal kernel runs on the same inputs for the
speedup.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-dense]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
WORKLOAD = "llama8b_s128k_bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops(cnt, hq, hkv, d, b, S):
    """Dense-equivalent and executed (block-level) attention FLOPs.

    executed: 4*d*(G*b)*b per (tile, kept block) -- diagonal blocks whole --
    plus 4*d*(G*b) per (tile, dropped block) for the mean-correction pseudo-key.
    dense-equivalent: 4*d*Hq*(S(S+1)/2), the causal query-key pairs."""
    G = hq // hkv
    nqb = cnt.shape[-1]
    kept = int(cnt.sum())
    visible = hkv * nqb * (nqb + 1) // 2
    dropped = visible - kept
    executed_attn = 4.0 * d * (G * b) * b * kept
    executed_corr = 4.0 * d * (G * b) * dropped
    dense_eq = 4.0 * d * hq * S * (S + 1) / 2
    dense_exec = 4.0 * d * (G * b) * b * visible
    return dict(kept=kept, visible=visible, sparsity=1.0 - kept / visible, executed=executed_attn + executed_corr,
                executed_attn=executed_attn, executed_corr=executed_corr, dense_eq=dense_eq, dense_exec=dense_exec)


def kernel_source_hash():
    """Hash of the HIP sources; HBM traffic read from profiles/ is reported only
    if it was measured on the same sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_long_scores_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per sparse-attention launch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, scaled by the copy-kernel calibration; None
    when the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "attn_sparse_128k_bf16_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(prob, hkv, b, tau, n_blocks=256, seed=0):
    """Time the float64 oracle on a bounded sample of the workload (about 10 s
    of CPU work): pooling and selection of KV group 0 over the whole sequence,
    attention of that group for a seeded sample of query blocks; extrapolated
    to one layer (all groups, all query blocks) in ms."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    S = prob.q.shape[0]
    G = prob.q.shape[1] // hkv
    t0 = time.perf_counter()
    q = prob.q[:, :G].float().numpy()
    k = prob.k[:, :1].float().numpy()
    v = prob.v[:, :1].float().numpy()
    t1 = time.perf_counter()
    qbar, kbar, vbar, n_k = A.pool(q, k, v, 1, b)
    geo = A.geometry(S, S, b)
    Sc = A.block_scores(qbar, kbar, geo.q_block_ids())
    kept, _ = A.select(Sc, geo.q_block_ids(), tau)
    t2 = time.perf_counter()
    rng = np.random.default_rng(seed)
    blocks = sorted(rng.choice(geo.nqb, size=n_blocks, replace=False).tolist())
    A.attend(q, k, v, kept, kbar, vbar, n_k, 1, b, 1 / math.sqrt(q.shape[2]), True, q_blocks=blocks)
    t3 = time.perf_counter()
    # attention work of a query block grows with its kept count; scale the
    # sampled time by total kept blocks / sampled kept blocks
    kept_rows = kept.sum(axis=2)[0]
    scale_attn = kept_rows.sum() / kept_rows[blocks].sum()
    per_layer = hkv * ((t2 - t1) + (t3 - t2) * scale_attn)
    return dict(value=per_layer * 1e3, unit="ms/layer (extrapolated)", cores=threads, kind="oracle",
                sample=f"float64 oracle on KV group 0: pool+select over all {geo.nqb} query blocks "
                       f"({t2 - t1:.1f} s) + attention of query blocks {blocks} ({t3 - t2:.1f} s); "
                       f"extrapolated x{hkv} groups and by kept-block count",
                measured_s=round(t3 - t1, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times), the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        x = torch.ones(1 << 28, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 << 28, "repeats": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (--gpus {args.gpus} requested): the hot path shards by KV head "
              "with no communication, so one GPU's share is what is measured here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_long_scores_amd as fp2
    import synth
    from tests.helpers import tau_table

    fp2.load()
    w = synth.WORKLOADS[WORKLOAD]
    S, hq, hkv, d, b = w["seqlen"], w["hq"], w["hkv"], w["d"], w["block"]
    tau = tau_table()[f"{WORKLOAD}@{w['sparsity']:.2f}"]["tau"]
    t0 = time.time()
    prob = synth.make_problem(w["kind"], args.seed, S, hq, hkv, d, b)
    log(f"[bench] generated {WORKLOAD} in {time.time() - t0:.1f}s; tau={tau:.4f}")

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (prob.q, prob.k, prob.v))
    p = fp2.make_params(hq, hkv, d, b, tau=tau)
    nqb, nkb = fp2.fp2_num_q_blocks(S, S, b), fp2.fp2_num_k_blocks(S, b)
    idx = torch.empty((1, hkv, nqb, nkb), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, hkv, nqb), dtype=torch.int32, device=dev)
    pk = torch.empty((1, hkv, nkb, d), dtype=torch.float32, device=dev)
    pv = torch.empty_like(pk)
    ws = torch.empty(fp2.fp2_select_workspace_size(p, 1, S, S), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def select():
        st = fp2.fp2_select_blocks(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                   cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(), ws.data_ptr(), ws.numel(), sh)
        assert st == 0, fp2.last_error()

    def attend():
        st = fp2.fp2_sparse_prefill(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                    cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(), out.data_ptr(), None, sh)
        assert st == 0, fp2.last_error()

    for _ in range(args.warmup):
        select()
        attend()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        select()
        e1.record(stream)
        attend()
        e2.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    sel_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    att_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))
    step_ms = float(np.mean([e0.elapsed_time(e2) for e0, _, e2 in ev]))
    log(f"[bench] select {sel_ms:.3f} ms, attention {att_ms:.3f} ms, step {step_ms:.3f} ms (wall {wall_ms:.3f})")

    F = flops(cnt.cpu().numpy(), hq, hkv, d, b, S)
    res_dense = None
    if not args.no_dense:
        out_d = torch.empty_like(q)

        def dense():
            st = fp2.fp2_dense_prefill(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(), out_d.data_ptr(), None,
                                       sh)
            assert st == 0, fp2.last_error()
        dense()
        torch.cuda.synchronize()
        evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.dense_steps)]
        for a_, b_ in evd:
            a_.record(stream)
            dense()
            b_.record(stream)
        torch.cuda.synchronize()
        dense_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evd]))
        res_dense = dict(ms=round(dense_ms, 3), tflops=round(F["dense_exec"] / dense_ms / 1e9, 1),
                         frac_peak=round(F["dense_exec"] / dense_ms / 1e9 / PEAK_BF16_TFLOPS, 4))
        log(f"[bench] dense {dense_ms:.3f} ms")
        diff = (out_d.float() - out.float()).norm() / out_d.float().norm()
        res_dense["sparse_vs_dense_rel_l2"] = round(float(diff), 4)

    achieved = F["executed"] / att_ms / 1e9   # TFLOP/s
    cpu = None
    if not args.no_cpu:
        log("[bench] timing the float64 oracle on a bounded sample ...")
        cpu = cpu_baseline(prob, hkv, b, tau)
        log(f"[bench] cpu baseline {cpu['value']:.0f} ms/layer ({cpu['measured_s']} s measured)")

    line = {
        "metric": "prefill-attn ms/layer @128K, eff. TFLOPS vs MFMA peak, speedup vs own dense",
        "value": round(step_ms, 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded planted-retrieval generator with RoPE; no dataset)",
        "config": {"workload": WORKLOAD, "seq_len": S, "batch": 1, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": b, "tau": round(tau, 5), "mean_correction": True,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": "attn_kernel<128,128> (fp2_sparse_prefill)"},
        "cpu_baseline": cpu,
        "breakdown": {
            "select_ms": round(sel_ms, 3),
            "sparse_attn_ms": round(att_ms, 3),
            "wall_ms_per_step": round(wall_ms, 3),
            "block_sparsity": round(F["sparsity"], 4),
            "kept_blocks": F["kept"],
            "executed_tflop": round(F["executed"] / 1e12, 3),
            "dense_equiv_tflop": round(F["dense_eq"] / 1e12, 3),
            "eff_tflops_dense_equiv": round(F["dense_eq"] / step_ms / 1e9, 1),
            "eff_tflops_executed_attn": round(achieved, 1),
            "dense": res_dense,
            "speedup_vs_dense": round(res_dense["ms"] / step_ms, 2) if res_dense else None,
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
