"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds none of the attention method's arithmetic: it draws
normals, plants structure, applies RoPE, rounds to bf16, quantizes to e4m3
with per-head amax scales (the FP8 inputs of the workload are quantized
upstream of the attention operator) and lays K/V out in a paged cache.  Both
the HIP library's callers and the oracle's callers take their inputs from
here; neither side's code lives here.

Reproducibility: every tensor is drawn in row chunks of ``CHUNK`` positions,
chunk c of tensor t of stream s from ``numpy.random.default_rng([seed, s, t,
c])`` (PCG64), so any range of positions regenerates identically without
drawing the rest.  Normals are drawn in float32, RoPE is applied in float32
with float64 angle tables, and the result is rounded to bf16 (RNE).
"""

from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1024
ROPE_BASE = 500000.0


def to_bf16(x):
    """float32 ndarray -> torch.bfloat16 (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _normals(seed, stream, tensor, start, stop, width):
    """Standard normals for positions [start, stop), shape [stop-start, width]."""
    out = np.empty((stop - start, width), dtype=np.float32)
    c0 = start // CHUNK
    c1 = -(-stop // CHUNK)
    for c in range(c0, c1):
        rng = np.random.default_rng([seed, stream, tensor, c])
        blk = rng.standard_normal((CHUNK, width), dtype=np.float32)
        a = max(start, c * CHUNK)
        b = min(stop, (c + 1) * CHUNK)
        out[a - start:b - start] = blk[a - c * CHUNK:b - c * CHUNK]
    return out


def rope_(x, positions, base=ROPE_BASE):
    """In-place rotate-half RoPE on x [n, H, d] (float32) at ``positions``.

    theta_f = base^(-2f/d), f < d/2; pairs (x[f], x[f + d/2]) rotate by
    position * theta_f.  No frequency rescaling."""
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    step = 8192
    for a in range(0, x.shape[0], step):
        ang = np.outer(positions[a:a + step].astype(np.float64), theta)
        cos = np.cos(ang).astype(np.float32)[:, None, :]
        sin = np.sin(ang).astype(np.float32)[:, None, :]
        x1 = x[a:a + step, :, :half].copy()
        x2 = x[a:a + step, :, half:]
        x[a:a + step, :, :half] = x1 * cos - x2 * sin
        x[a:a + step, :, half:] = x2 * cos + x1 * sin
    return x


@dataclass
class Planted:
    """Structure of the planted generator for one sequence."""
    u: np.ndarray          # [Hkv, d] unit vectors
    hot: list              # per KV head: sorted hot key-block ids


def planted_structure(seed, stream, seqlen, hkv, d, block, hot_frac=0.05):
    rng = np.random.default_rng([seed, stream, 0xFFFF])
    nb = -(-seqlen // block)
    u = rng.standard_normal((hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    n_hot = int(round(hot_frac * nb))
    hot = [np.sort(rng.choice(nb, size=n_hot, replace=False)) for _ in range(hkv)]
    return Planted(u.astype(np.float32), hot)


def planted_rows(seed, stream, seqlen, hq, hkv, d, block, which, start, stop,
                 k_shift=3.0, q_shift=1.5, rope_base=ROPE_BASE):
    """Rows [start, stop) of Q, K or V (``which``) of the planted generator.

    Per KV head h: unit vector u_h; round(0.05 * nblocks) hot key blocks; K is
    N(0,1) plus 3*u_h on hot blocks; every query head of group h is N(0,1)
    plus 1.5*u_h; the plant comes first, then RoPE at the absolute position
    (so it rotates the planted component); V is N(0,1)."""
    st = planted_structure(seed, stream, seqlen, hkv, d, block)
    pos = np.arange(start, stop)
    if which == "v":
        return _normals(seed, stream, 3, start, stop, hkv * d).reshape(-1, hkv, d)
    if which == "k":
        x = _normals(seed, stream, 2, start, stop, hkv * d).reshape(-1, hkv, d)
        blk = pos // block
        for h in range(hkv):
            rows = np.isin(blk, st.hot[h])
            x[rows, h, :] += k_shift * st.u[h]
    elif which == "q":
        g = hq // hkv
        x = _normals(seed, stream, 1, start, stop, hq * d).reshape(-1, hq, d)
        x += q_shift * np.repeat(st.u, g, axis=0)[None]
    else:
        raise ValueError(which)
    return rope_(x, pos, rope_base)


def iid_rows(seed, stream, heads, d, which, start, stop):
    """Rows of an i.i.d. N(0,1) tensor (no structure, no RoPE)."""
    t = {"q": 1, "k": 2, "v": 3}[which]
    return _normals(seed, stream, t, start, stop, heads * d).reshape(-1, heads, d)


@dataclass
class Problem:
    """One contiguous-layout problem, batch 1: bf16 tensors on the CPU."""
    q: torch.Tensor        # [Sq, Hq, d]
    k: torch.Tensor        # [Sk, Hkv, d]
    v: torch.Tensor        # [Sk, Hkv, d]
    block: int
    meta: dict = field(default_factory=dict)


def make_problem(kind, seed, seqlen_k, hq, hkv, d, block, seqlen_q=None,
                 stream=0):
    """kind 'iid' or 'planted'.  Q covers the last ``seqlen_q`` positions."""
    seqlen_q = seqlen_k if seqlen_q is None else seqlen_q
    P = seqlen_k - seqlen_q
    if kind == "iid":
        q = iid_rows(seed, stream, hq, d, "q", P, seqlen_k)
        k = iid_rows(seed, stream, hkv, d, "k", 0, seqlen_k)
        v = iid_rows(seed, stream, hkv, d, "v", 0, seqlen_k)
    elif kind == "planted":
        q = planted_rows(seed, stream, seqlen_k, hq, hkv, d, block, "q", P, seqlen_k)
        k = planted_rows(seed, stream, seqlen_k, hq, hkv, d, block, "k", 0, seqlen_k)
        v = planted_rows(seed, stream, seqlen_k, hq, hkv, d, block, "v", 0, seqlen_k)
    else:
        raise ValueError(kind)
    return Problem(to_bf16(q), to_bf16(k), to_bf16(v), block,
                   dict(kind=kind, seed=seed, stream=stream))


# ---------------------------------------------------------------- FP8 inputs

E4M3_MAX = 448.0


def e4m3_scales(x, head_axis):
    """Per-head amax calibration: scale_h = amax_h / 448 (1 if amax_h = 0)."""
    xf = x.float()
    dims = [a for a in range(xf.dim()) if a != head_axis]
    amax = xf.abs().amax(dim=dims)
    return torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()


def quantize_e4m3(x, head_axis, scale=None):
    """code = RNE(x / scale_h) saturated to +-448, with per-head scales from
    e4m3_scales unless given.  Returns (uint8 codes tensor, float32 scales
    tensor).  The cast is torch's float8_e4m3fn conversion."""
    xf = x.float()
    if scale is None:
        scale = e4m3_scales(xf, head_axis)
    shape = [1] * xf.dim()
    shape[head_axis] = -1
    y = (xf / scale.reshape(shape)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.float().contiguous()


# ---------------------------------------------------------------- paged KV

@dataclass
class PagedBatch:
    q: torch.Tensor            # [total_q, Hq, d] packed new rows
    cu_seqlens_q: torch.Tensor # [n+1] int32
    seqlens_k: torch.Tensor    # [n] int32 (prefix + new chunk)
    k_cache: torch.Tensor      # [num_phys_pages, page, Hkv, d]
    v_cache: torch.Tensor
    page_table: torch.Tensor   # [n, max_pages_per_seq] int32
    page_size: int
    block: int
    seqs: list                 # per sequence: dict(q, k, v) logical bf16 tensors
    canary_pages: np.ndarray
    q_scale: torch.Tensor = None  # fp8 batches: per-head scales [Hq], [Hkv], [Hkv]
    k_scale: torch.Tensor = None
    v_scale: torch.Tensor = None


def make_paged(seed, kv_lens, q_lens, hq, hkv, d, block, page_size=64,
               kind="planted", n_canary=64, fp8=False):
    """Continuous batch: sequence s has kv_lens[s] tokens in the cache, the
    last q_lens[s] of them new (query rows).  Sequence s is generated at its
    full length from stream s+1.  Physical pages are a seeded permutation of
    num_pages + n_canary pages; the canary pages hold NaN and are never
    referenced; unused page-table entries point at a canary page.
    fp8: q and the caches become e4m3 codes with per-head scales calibrated
    over the whole batch; each seqs entry also gets its codes (qc, kc, vc)."""
    n = len(kv_lens)
    pages_per = [-(-L // page_size) for L in kv_lens]
    num_pages = sum(pages_per)
    max_pages = max(pages_per)
    rng = np.random.default_rng([seed, 0xCAFE])
    perm = rng.permutation(num_pages + n_canary)
    canary = perm[num_pages:]
    k_cache = torch.full((num_pages + n_canary, page_size, hkv, d), float("nan"),
                         dtype=torch.bfloat16)
    v_cache = torch.full_like(k_cache, float("nan"))
    table = np.full((n, max_pages), canary[0], dtype=np.int32)
    seqs = []
    qs = []
    nxt = 0
    for s in range(n):
        L, Lq = kv_lens[s], q_lens[s]
        pr = make_problem(kind, seed, L, hq, hkv, d, block, seqlen_q=Lq, stream=s + 1)
        seqs.append(dict(q=pr.q, k=pr.k, v=pr.v))
        qs.append(pr.q)
        for pg in range(pages_per[s]):
            phys = int(perm[nxt])
            nxt += 1
            table[s, pg] = phys
            a = pg * page_size
            b = min(L, a + page_size)
            k_cache[phys, :b - a] = pr.k[a:b]
            v_cache[phys, :b - a] = pr.v[a:b]
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = torch.cat(qs, 0)
    scales = (None, None, None)
    if fp8:
        qsc = e4m3_scales(q, 1)
        ksc = e4m3_scales(torch.cat([x["k"] for x in seqs], 0), 1)
        vsc = e4m3_scales(torch.cat([x["v"] for x in seqs], 0), 1)
        q = quantize_e4m3(q, 1, qsc)[0]
        k_cache = quantize_e4m3(k_cache, 2, ksc)[0]   # NaN canaries stay NaN codes
        v_cache = quantize_e4m3(v_cache, 2, vsc)[0]
        for x in seqs:
            x["qc"] = quantize_e4m3(x["q"], 1, qsc)[0]
            x["kc"] = quantize_e4m3(x["k"], 1, ksc)[0]
            x["vc"] = quantize_e4m3(x["v"], 1, vsc)[0]
        scales = (qsc, ksc, vsc)
    return PagedBatch(q, torch.from_numpy(cu),
                      torch.tensor(kv_lens, dtype=torch.int32), k_cache, v_cache,
                      torch.from_numpy(table), page_size, block, seqs, canary, *scales)


# ---------------------------------------------------------------- workloads

WORKLOADS = {
    # name: dict(kind, seqlen, hq, hkv, d, block, target_sparsity)
    "tiny_gqa4_d64_s1024": dict(kind="iid", seqlen=1024, hq=4, hkv=1, d=64,
                                block=64, tau=2.0, out="fp32"),
    "llama8b_s32k_bf16": dict(kind="planted", seqlen=32768, hq=32, hkv=8, d=128,
                              block=128, sparsity=0.70, out="bf16"),
    "llama8b_s128k_bf16": dict(kind="planted", seqlen=131072, hq=32, hkv=8,
                               d=128, block=128, sparsity=0.80, out="bf16"),
    "llama8b_s128k_fp8": dict(kind="planted", seqlen=131072, hq=32, hkv=8,
                              d=128, block=128, sparsity=(0.80, 0.85, 0.90),
                              out="bf16", fp8=True),
    "paged_batch6": dict(kind="planted", kv_lens=[4096, 8192, 16384, 32768, 65536, 131072],
                         q_lens=[4096, 8192, 16384, 32768, 8192, 16384], hq=32,
                         hkv=8, d=128, block=128, page_size=64, sparsity=0.80,
                         out="bf16"),
}
