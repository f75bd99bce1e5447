"""Write tests/golden/tau_table.json: the threshold tau of each workload.

Each workload names a target block sparsity; tau is found by bisection on the
oracle's float64 block scores of the seeded synthetic inputs (pool -> score
-> select), so that 1 - kept/visible lands within 0.5% of the target.  Only
``synth`` (inputs) and ``oracle`` are used.  Run from the repository root:

    python tests/golden/make_tau_table.py
"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import attention as A  # noqa: E402


def bisect_tau(scores, target, iters=60):
    """scores: list of (S, ids); returns (tau, achieved sparsity)."""
    def sp(tau):
        kept = 0
        vis = 0
        for S, ids in scores:
            k, _ = A.select(S, ids, tau)
            kept += k.sum()
            vis += S.shape[0] * int(np.sum(ids + 1))
        return 1.0 - kept / vis
    lo, hi = 0.0, 1.0
    while sp(hi) > target:
        hi *= 2
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if sp(mid) > target:
            lo = mid
        else:
            hi = mid
    tau = hi
    return tau, sp(tau)


def scores_for(q, k, v, hkv, block):
    qbar, kbar, vbar, n_k = A.pool(q, k, v, hkv, block)
    geo = A.geometry(q.shape[0], k.shape[0], block)
    return A.block_scores(qbar, kbar, geo.q_block_ids()), geo.q_block_ids()


def f32(t):
    return t.float().numpy()


def main(seed=0):
    out = {"seed": seed, "generated_by": "tests/golden/make_tau_table.py", "entries": {}}
    W = synth.WORKLOADS
    for name in ["llama8b_s32k_bf16", "llama8b_s128k_bf16", "llama8b_s128k_fp8"]:
        w = W[name]
        t0 = time.time()
        pr = synth.make_problem(w["kind"], seed, w["seqlen"], w["hq"], w["hkv"], w["d"], w["block"])
        if w.get("fp8"):
            qc, qs = synth.quantize_e4m3(pr.q, 1)
            kc, ks = synth.quantize_e4m3(pr.k, 1)
            vc, vs = synth.quantize_e4m3(pr.v, 1)
            q = oracle.dequantize(qc.numpy(), qs.numpy(), 1)
            k = oracle.dequantize(kc.numpy(), ks.numpy(), 1)
            v = oracle.dequantize(vc.numpy(), vs.numpy(), 1)
        else:
            q, k, v = f32(pr.q), f32(pr.k), f32(pr.v)
        S, ids = scores_for(q, k, v, w["hkv"], w["block"])
        targets = w["sparsity"] if isinstance(w["sparsity"], tuple) else (w["sparsity"],)
        for tgt in targets:
            tau, sp = bisect_tau([(S, ids)], tgt)
            out["entries"][f"{name}@{tgt:.2f}"] = dict(tau=tau, sparsity=sp, target=tgt)
            print(name, tgt, tau, sp, f"{time.time() - t0:.1f}s", flush=True)
        del q, k, v, pr
    w = W["paged_batch6"]
    pb = synth.make_paged(seed, w["kv_lens"], w["q_lens"], w["hq"], w["hkv"], w["d"],
                          w["block"], w["page_size"])
    sc = [scores_for(f32(s["q"]), f32(s["k"]), f32(s["v"]), w["hkv"], w["block"]) for s in pb.seqs]
    tau, sp = bisect_tau(sc, w["sparsity"])
    out["entries"][f"paged_batch6@{w['sparsity']:.2f}"] = dict(tau=tau, sparsity=sp, target=w["sparsity"])
    print("paged", tau, sp, flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tau_table.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print("wrote", path)


if __name__ == "__main__":
    main()
