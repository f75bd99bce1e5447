"""Shared helpers of the GPU parity tests: input staging, mask decoding,
error metrics.  No attention arithmetic lives here (that is the oracle's and
the library's)."""

import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

BF16_REL_L2 = 1e-2     # output tolerance, bf16 path (relative L2 error)
BF16_MAX_ABS = 2e-2    # output tolerance, bf16 path (max abs error)
FP8_REL_L2 = 5e-2      # output tolerance, fp8 path
MASK_BAND = 1e-3       # blocks whose score is within this of the threshold may differ


def tau_table():
    with open(os.path.join(GOLDEN, "tau_table.json")) as f:
        return json.load(f)["entries"]


def f64(t):
    """bf16/fp32 torch tensor (any device) -> float64 numpy (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


BF16_LSE_ABS = 2e-2    # LSE tolerance, bf16 path
# LSE tolerance, fp8 path: P is stored as log-linear e4m3 codes, each within a
# factor exp(+-0.0728) of its exact value (tests/test_tolerances.py), so a row
# dominated by one key can have its normaliser off by up to 0.0728
FP8_LSE_ABS = 0.08


# One record per check_blocks call (label, pairs checked, worst and last-block
# errors, tolerance), printed by the session's terminal summary so that the
# per-block figures show in quiet runs too.
PARITY_LOG = []


def block_errors(o, O, geo, hkv, blocks=None, lse=None, L=None):
    """Errors of every (query block, KV head) pair on its own: the rows of
    query block i (absolute id) and the G query heads of KV head h.
    o, O [Sq, Hq, d]; lse, L [Hq, Sq] (optional).  Returns a list of dicts
    with block, head, rows, rel_l2, max_abs and lse_err."""
    o = np.asarray(o, np.float64).reshape(O.shape)
    G = O.shape[1] // hkv
    ids = geo.q_block_ids() if blocks is None else blocks
    res = []
    for i in ids:
        r0, r1 = geo.q_rows(int(i))
        for h in range(hkv):
            a, b = o[r0:r1, h * G:(h + 1) * G], O[r0:r1, h * G:(h + 1) * G]
            e = dict(block=int(i), head=h, rows=r1 - r0, rel_l2=rel_l2(a, b), max_abs=max_abs(a, b),
                     finite=bool(np.isfinite(a).all()), lse_err=0.0)
            if lse is not None:
                e["lse_err"] = float(np.abs(np.asarray(lse, np.float64)[h * G:(h + 1) * G, r0:r1]
                                            - L[h * G:(h + 1) * G, r0:r1]).max())
            res.append(e)
    return res


def check_blocks(o, O, geo, hkv, fp8=False, blocks=None, lse=None, L=None, label="parity", rel_tol=None):
    """Hold every (query block, KV head) pair to the output tolerance on its
    own (rel-L2 <= 1e-2 and max-abs <= 2e-2 in bf16, rel-L2 <= 5e-2 in fp8;
    LSE within 2e-2 / 0.08), so that large outputs of one block (the first
    query blocks attend to few keys) cannot hide the error of another.
    Prints the worst pair and the last block; returns the error list."""
    errs = block_errors(o, O, geo, hkv, blocks, lse, L)
    tol = rel_tol if rel_tol is not None else (FP8_REL_L2 if fp8 else BF16_REL_L2)
    lse_tol = FP8_LSE_ABS if fp8 else BF16_LSE_ABS
    wr = max(errs, key=lambda e: e["rel_l2"])
    wa = max(errs, key=lambda e: e["max_abs"])
    last = max(e["block"] for e in errs)
    lastr = max(e["rel_l2"] for e in errs if e["block"] == last)
    msg = (f"[{label}] {len(errs)} (q-block, kv-head) pairs: worst rel_l2 {wr['rel_l2']:.2e} (block {wr['block']} "
           f"head {wr['head']}), worst max_abs {wa['max_abs']:.2e} (block {wa['block']} head {wa['head']}), "
           f"last block {last} rel_l2 {lastr:.2e}")
    if lse is not None:
        msg += f", worst lse_err {max(e['lse_err'] for e in errs):.2e}"
    print(msg, flush=True)
    PARITY_LOG.append(dict(label=label, pairs=len(errs), worst_rel_l2=wr["rel_l2"], worst_block=wr["block"],
                           worst_head=wr["head"], worst_max_abs=wa["max_abs"], last_block=last,
                           last_rel_l2=lastr, tol=tol, fp8=fp8,
                           worst_lse=max(e["lse_err"] for e in errs) if lse is not None else None))
    bad = [e for e in errs if not (e["finite"] and e["rel_l2"] < tol and (fp8 or e["max_abs"] < BF16_MAX_ABS)
                                   and e["lse_err"] < lse_tol)]
    assert not bad, f"{len(bad)} of {len(errs)} (block, head) pairs over tolerance, first: {bad[:4]}"
    return errs


def kept_from_lists(idx, cnt, nkb):
    """GPU (block_idx, block_cnt) of one sequence [Hkv, nqb, nkb] / [Hkv, nqb]
    -> bool mask; also checks the lists are strictly ascending."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    H, nq = cnt.shape
    kept = np.zeros((H, nq, nkb), dtype=bool)
    for h in range(H):
        for il in range(nq):
            c = int(cnt[h, il])
            lst = idx[h, il, :c]
            assert c >= 1, (h, il)
            assert np.all(np.diff(lst) > 0), f"list of row {(h, il)} not strictly ascending"
            assert lst.min() >= 0 and lst.max() < nkb
            kept[h, il, lst] = True
    return kept


def assert_mask_matches(kept_gpu, kept_ref, S, thr, band=MASK_BAND):
    """Bit-exact outside the near-threshold band; returns the number of
    (legitimate) flips inside the band."""
    from oracle import score_band_mask
    inband = score_band_mask(S, thr, band)
    diff = kept_gpu != kept_ref
    bad = diff & ~inband
    assert not bad.any(), f"{int(bad.sum())} mask entries differ outside the +-{band} band, first at {np.argwhere(bad)[:5]}"
    return int((diff & inband).sum())


def to_dev(*ts, device="cuda"):
    return [t.to(device) for t in ts]
