"""Float64 oracle: pool -> block scores -> max-threshold select -> attend.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may call it).

One call handles ONE sequence in "SHD" layout: q [Sq, Hq, d], k and v
[Sk, Hkv, d].  Query row r sits at absolute position p = P + r with
P = Sk - Sq (a chunked prefill over a cached prefix when P > 0).  Query head
hq reads KV head hq // G with G = Hq / Hkv (grouped-query attention, [EXP]
§2.2).  Blocks are numbered by absolute position: key block j holds keys
[j*b, (j+1)*b) and query block i holds the query rows whose positions fall in
[i*b, (i+1)*b).

Method (the steps in the pages' order):

1. Pattern discovery ([ABS]: "instantaneous pattern discovery"; [NEWS]).
   Reading: block mean-pooling.  qbar_i is the mean of Q over the G query
   heads of a KV group and the rows of query block i present in the call;
   kbar_j, vbar_j are the means of K and V over the keys of block j.  The
   block score is the unscaled dot product S_ij = <qbar_i, kbar_j>, 0 <= j <= i.
2. Max-based dynamic thresholding ([ABS]).  m_i = max_{0<=j<=i} S_ij; block j
   is kept iff S_ij >= m_i - tau; the sink block 0 and the diagonal block i
   are always kept.  Supp(q) ([EXP] §2.1) is the kept set of q's block.
3. Block-sparse attention ([EXP] §2.1, V1): each query attends only to the
   keys of its kept blocks, causally (key position <= query position).
4. Mean correction ([EXP] §2.1 and [SCR] §4 scene-4, formula Out_q^V2;
   [ABS] "mean correction term").  Reading of the schematic formula: every
   dropped block j enters the same softmax as ONE pseudo-key with logit
   scale*<q, kbar_j> + ln n_j (n_j keys in block j) and value vbar_j.  That
   is exact when all keys of a dropped block are equal, and in general it
   equals  O = O_supp - mu_q * (O_supp - Vbar_drop)  with mu_q the softmax
   mass of the dropped blocks and Vbar_drop their mass-weighted mean value:
   the ingredients of Out_q^V2 (see ``correction_split``).
5. Output O = (sum_c e^{l_c - M} v_c + sum_j e^{l^_j - M} vbar_j) / (sum of the
   same weights); LSE = M + ln(denominator).
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Geometry:
    """Block geometry of one sequence (absolute block numbering)."""
    seqlen_q: int
    seqlen_k: int
    block: int
    q_offset: int      # P = Sk - Sq
    first_qblock: int  # absolute index of the first query block touched
    nqb: int           # number of query blocks touched by the call
    nkb: int           # number of key blocks = ceil(Sk / b)

    def q_block_ids(self):
        return np.arange(self.first_qblock, self.first_qblock + self.nqb)

    def q_rows(self, i):
        """Local query rows [r0, r1) of absolute query block i."""
        p0 = max(i * self.block, self.q_offset)
        p1 = min((i + 1) * self.block, self.q_offset + self.seqlen_q)
        return p0 - self.q_offset, p1 - self.q_offset

    def k_rows(self, j):
        return j * self.block, min((j + 1) * self.block, self.seqlen_k)


def geometry(seqlen_q, seqlen_k, block):
    if not (0 < seqlen_q <= seqlen_k):
        raise ValueError("need 0 < seqlen_q <= seqlen_k")
    P = seqlen_k - seqlen_q
    first = P // block
    last = (seqlen_k - 1) // block
    nkb = -(-seqlen_k // block)
    return Geometry(seqlen_q, seqlen_k, block, P, first, last - first + 1, nkb)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def pool(q, k, v, num_kv_heads, block):
    """Step 1: block means.

    Returns qbar [Hkv, nqb, d] (mean over the G heads of each group and the
    present rows of each query block), kbar and vbar [Hkv, nkb, d], and
    n_k [nkb] (keys per key block).
    """
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    G = Hq // num_kv_heads
    geo = geometry(Sq, Sk, block)
    qbar = np.empty((num_kv_heads, geo.nqb, d))
    for il, i in enumerate(geo.q_block_ids()):
        r0, r1 = geo.q_rows(i)
        blk = _f64(q[r0:r1]).reshape(r1 - r0, num_kv_heads, G, d)
        qbar[:, il, :] = blk.mean(axis=(0, 2))
    kbar = np.empty((num_kv_heads, geo.nkb, d))
    vbar = np.empty((num_kv_heads, geo.nkb, d))
    n_k = np.empty(geo.nkb, dtype=np.int64)
    for j in range(geo.nkb):
        c0, c1 = geo.k_rows(j)
        kbar[:, j, :] = _f64(k[c0:c1]).mean(axis=0)
        vbar[:, j, :] = _f64(v[c0:c1]).mean(axis=0)
        n_k[j] = c1 - c0
    return qbar, kbar, vbar, n_k


def block_scores(qbar, kbar, q_block_ids):
    """Step 1 (scores): S[h, il, j] = <qbar[h, il], kbar[h, j]> for j <= i, NaN above."""
    S = np.einsum("hid,hjd->hij", qbar, kbar)
    j = np.arange(kbar.shape[1])
    visible = j[None, :] <= np.asarray(q_block_ids)[:, None]
    return np.where(visible[None], S, np.nan)


def select(S, q_block_ids, tau):
    """Step 2: kept[h, il, j] (bool) and the thresholds m_i - tau [Hkv, nqb]."""
    ids = np.asarray(q_block_ids)
    m = np.nanmax(S, axis=2)
    thr = m - tau
    with np.errstate(invalid="ignore"):
        kept = S >= thr[:, :, None]
    kept = kept & ~np.isnan(S)
    kept[:, :, 0] = True
    kept[:, np.arange(len(ids)), ids] = True
    return kept, thr


def pool_q_heads(q, seqlen_k, block):
    """Per-query-head block means (selection variants "union" and "max"): qbar_heads
    [Hq, nqb, d], each the mean over the rows of block i present in this call."""
    Sq, Hq, d = q.shape
    geo = geometry(Sq, seqlen_k, block)
    out = np.empty((Hq, geo.nqb, d))
    for il, i in enumerate(geo.q_block_ids()):
        r0, r1 = geo.q_rows(i)
        out[:, il, :] = _f64(q[r0:r1]).mean(axis=0)
    return out


def select_union(qbar_heads, kbar, q_block_ids, tau):
    """Selection variant "union" (a reading for per-query-head masks under
    GQA packing, whose K/V tile is shared by the group): every query head
    applies the max-threshold rule to its own scores <qbar_hq, kbar_j>, and a
    key block is kept for the group if any of its heads keeps it (plus the
    sink and diagonal blocks).  Returns kept [Hkv, nqb, nkb], the per-head
    scores S [Hq, nqb, nkb] and thresholds [Hq, nqb]."""
    Hq = qbar_heads.shape[0]
    Hkv = kbar.shape[0]
    G = Hq // Hkv
    kbar_heads = np.repeat(kbar, G, axis=0)          # query head hq reads group hq // G
    S = block_scores(qbar_heads, kbar_heads, q_block_ids)
    kept_heads, thr = select(S, q_block_ids, tau)
    kept = kept_heads.reshape(Hkv, G, *kept_heads.shape[1:]).any(axis=1)
    return kept, S, thr


def select_head_max(qbar_heads, kbar, q_block_ids, tau):
    """Selection variant "max" (another reading of how a GQA group's heads
    share one mask, [EXP] §2.2 PackGQA with the selection of §2.1): the
    group's block score is the largest of its query heads' scores,
    S_ij = max_{hq in group} <qbar_hq,i, kbar_j>, and the max-threshold rule
    of step 2 runs on that score (plus the sink and diagonal blocks).  The
    group-mean reading averages the same per-head scores instead, since the
    score is linear in qbar.  Returns kept [Hkv, nqb, nkb], the group scores
    S [Hkv, nqb, nkb] and thresholds [Hkv, nqb]."""
    Hq = qbar_heads.shape[0]
    Hkv = kbar.shape[0]
    G = Hq // Hkv
    S_heads = block_scores(qbar_heads, np.repeat(kbar, G, axis=0), q_block_ids)
    S = S_heads.reshape(Hkv, G, *S_heads.shape[1:]).max(axis=1)   # NaN (invisible) stays NaN
    kept, thr = select(S, q_block_ids, tau)
    return kept, S, thr


def union_band_mask(S_heads, thr_heads, num_kv_heads, band=1e-3):
    """score_band_mask of the union selection: a group's block may differ
    between two correct selections where any of its heads scores within
    ``band`` of that head's threshold."""
    b = score_band_mask(S_heads, thr_heads, band)
    G = b.shape[0] // num_kv_heads
    return b.reshape(num_kv_heads, G, *b.shape[1:]).any(axis=1)


def score_band_mask(S, thr, band=1e-3):
    """True where a block's score lies within ``band`` of its row threshold:
    the only places where two correct selections may differ."""
    with np.errstate(invalid="ignore"):
        return np.abs(S - thr[:, :, None]) <= band


def sparsity(kept, q_block_ids):
    """1 - kept / visible over the causally visible block pairs j <= i."""
    ids = np.asarray(q_block_ids)
    visible = kept.shape[0] * int(np.sum(ids + 1))
    return 1.0 - kept.sum() / visible


def _tile_terms(q, k, v, kept_row, kbar_h, vbar_h, n_k, geo, h, i, G, scale,
                mean_correction):
    """Logits and values of one (KV head h, query block i) tile.

    Returns (rows, Qt, real logits [R, C] with -inf where masked, real values
    [C, d], pseudo logits [R, D], pseudo values [D, d])."""
    r0, r1 = geo.q_rows(i)
    d = q.shape[2]
    nr = r1 - r0
    Qt = _f64(q[r0:r1, h * G:(h + 1) * G, :]).reshape(nr * G, d)
    pos = (np.arange(r0, r1) + geo.q_offset).repeat(G)       # row-major (r, g)
    kept_j = np.flatnonzero(kept_row)
    keys = np.concatenate([np.arange(*geo.k_rows(j)) for j in kept_j])
    Kc = _f64(k[keys, h, :])
    Vc = _f64(v[keys, h, :])
    logits = scale * (Qt @ Kc.T)
    logits = np.where(keys[None, :] <= pos[:, None], logits, -np.inf)
    if mean_correction:
        dropped = np.flatnonzero(~kept_row[: i + 1])
    else:
        dropped = np.zeros(0, dtype=np.int64)
    plog = scale * (Qt @ kbar_h[dropped].T) + np.log(n_k[dropped])[None, :]
    return (r0, r1), Qt, logits, Vc, plog, vbar_h[dropped]


def attend(q, k, v, kept, kbar, vbar, n_k, num_kv_heads, block, scale,
           mean_correction=True, q_blocks=None):
    """Steps 3-5.  Returns O [Sq, Hq, d] and LSE [Hq, Sq] in float64.

    ``q_blocks`` (absolute ids) limits the work to those query blocks; other
    rows are left NaN.  ``kept`` is [Hkv, nqb, nkb] bool (any mask that holds
    the diagonal block works, e.g. a GPU-exported one)."""
    Sq, Hq, d = q.shape
    G = Hq // num_kv_heads
    geo = geometry(Sq, k.shape[0], block)
    O = np.full((Sq, Hq, d), np.nan)
    LSE = np.full((Hq, Sq), np.nan)
    ids = geo.q_block_ids() if q_blocks is None else np.asarray(q_blocks)
    for i in ids:
        il = i - geo.first_qblock
        for h in range(num_kv_heads):
            (r0, r1), _, lg, Vc, plg, pv = _tile_terms(
                q, k, v, kept[h, il], kbar[h], vbar[h], n_k, geo, h, i, G,
                scale, mean_correction)
            M = np.maximum(lg.max(axis=1), plg.max(axis=1, initial=-np.inf))
            E = np.exp(lg - M[:, None])
            Ep = np.exp(plg - M[:, None])
            den = E.sum(axis=1) + Ep.sum(axis=1)
            num = E @ Vc + Ep @ pv
            o = (num / den[:, None]).reshape(r1 - r0, G, d)
            O[r0:r1, h * G:(h + 1) * G, :] = o
            LSE[h * G:(h + 1) * G, r0:r1] = (M + np.log(den)).reshape(r1 - r0, G).T
    return O, LSE


def correction_split(q, k, v, kept, kbar, vbar, n_k, num_kv_heads, block,
                     scale, i):
    """The Out_q^V2 ingredients for query block i, computed apart from the fold.

    Returns (O_supp, Vbar_drop, mu) for every (row, head) of the block:
    O_supp is softmax attention normalised over Supp(q) only, Vbar_drop the
    pseudo-key-weighted mean of the dropped blocks' vbar, and mu the share of
    the softmax mass that the dropped blocks carry.  The fold in ``attend``
    must equal O_supp - mu * (O_supp - Vbar_drop)."""
    Sq, Hq, d = q.shape
    G = Hq // num_kv_heads
    geo = geometry(Sq, k.shape[0], block)
    il = i - geo.first_qblock
    outs = []
    for h in range(num_kv_heads):
        _, _, lg, Vc, plg, pv = _tile_terms(q, k, v, kept[h, il], kbar[h],
                                            vbar[h], n_k, geo, h, i, G, scale,
                                            True)
        M = np.maximum(lg.max(axis=1), plg.max(axis=1, initial=-np.inf))
        Es = np.exp(lg - M[:, None])
        Ed = np.exp(plg - M[:, None])
        Ws = Es.sum(axis=1)
        Wd = Ed.sum(axis=1)
        O_supp = (Es @ Vc) / Ws[:, None]
        Vdrop = (Ed @ pv) / np.where(Wd > 0, Wd, 1.0)[:, None]
        mu = Wd / (Ws + Wd)
        outs.append((O_supp, Vdrop, mu))
    return outs


def dense_attention(q, k, v, num_kv_heads, scale, rows=None):
    """Textbook causal attention softmax(scale * Q K^T) V ([EXP] §1.1), per
    query head, with query row r at position Sk - Sq + r.  ``rows`` limits the
    rows computed (others NaN).  Returns O [Sq, Hq, d] and LSE [Hq, Sq]."""
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    G = Hq // num_kv_heads
    P = Sk - Sq
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    O = np.full((Sq, Hq, d), np.nan)
    LSE = np.full((Hq, Sq), np.nan)
    for hq in range(Hq):
        h = hq // G
        Qr = _f64(q[rows, hq, :])
        L = scale * (Qr @ _f64(k[:, h, :]).T)
        L = np.where(np.arange(Sk)[None, :] <= (rows + P)[:, None], L, -np.inf)
        M = L.max(axis=1)
        E = np.exp(L - M[:, None])
        s = E.sum(axis=1)
        O[rows, hq, :] = (E @ _f64(v[:, h, :])) / s[:, None]
        LSE[hq, rows] = M + np.log(s)
    return O, LSE


def sparse_prefill(q, k, v, num_kv_heads, block, tau, scale=None,
                   mean_correction=True, q_blocks=None, select_mode="mean"):
    """The whole pipeline on one sequence: pool, score, select, attend.
    select_mode "mean": one query mean per GQA group (the default reading);
    "union": per-query-head selection, united over the group (S and thr are
    then per query head); "max": the group's score is the largest of its
    heads' scores (S and thr per KV head, as for "mean")."""
    d = q.shape[2]
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    geo = geometry(q.shape[0], k.shape[0], block)
    qbar, kbar, vbar, n_k = pool(q, k, v, num_kv_heads, block)
    if select_mode == "union":
        qbar = pool_q_heads(q, k.shape[0], block)
        kept, S, thr = select_union(qbar, kbar, geo.q_block_ids(), tau)
    elif select_mode == "max":
        qbar = pool_q_heads(q, k.shape[0], block)
        kept, S, thr = select_head_max(qbar, kbar, geo.q_block_ids(), tau)
    elif select_mode == "mean":
        S = block_scores(qbar, kbar, geo.q_block_ids())
        kept, thr = select(S, geo.q_block_ids(), tau)
    else:
        raise ValueError(f"unknown select_mode {select_mode!r}")
    O, LSE = attend(q, k, v, kept, kbar, vbar, n_k, num_kv_heads, block,
                    scale, mean_correction, q_blocks)
    return dict(geo=geo, qbar=qbar, kbar=kbar, vbar=vbar, n_k=n_k, S=S,
                kept=kept, thr=thr, O=O, LSE=LSE, scale=scale)
