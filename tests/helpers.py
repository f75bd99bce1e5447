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
