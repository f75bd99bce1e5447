"""Pins of the float64 oracle against things other than itself (CPU only).

Each test pins one part of the oracle against brute force written as
explicit loops, a textbook definition, a closed-form special case, an
invariant, or a library routine, so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong pooling
axis, a wrong GQA head mapping) fails at least one of them.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

_STATE = {"rng": np.random.default_rng(12345)}


@pytest.fixture(autouse=True)
def _per_test_generator(request):
    """Each test draws from its own generator, seeded by its name, so the
    inputs a test sees do not depend on which tests ran before it."""
    _STATE["rng"] = np.random.default_rng(zlib.crc32(request.node.name.encode()))


def _rand(*shape, scale=1.0):
    return _STATE["rng"].standard_normal(shape) * scale


# ------------------------------------------------------------------ e4m3

def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.isnan(ours).sum() == 2          # S.1111.111 only


def test_e4m3_format_landmarks():
    dec = oracle.e4m3_decode
    assert dec(np.uint8(0x38)) == 1.0
    assert dec(np.uint8(0x7E)) == 448.0          # largest finite
    assert dec(np.uint8(0x01)) == 2.0 ** -9      # smallest subnormal
    assert dec(np.uint8(0x08)) == 2.0 ** -6      # smallest normal
    assert dec(np.uint8(0xC5)) == -3.25
    assert np.signbit(dec(np.uint8(0x80))) and dec(np.uint8(0x80)) == 0.0


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals)
    # -0 encodes as +0 (both decode to zero); every other code comes back
    nz = vals != 0
    assert np.array_equal(back[nz], codes[nz])
    assert np.all(oracle.e4m3_decode(back[~nz]) == 0)


def test_e4m3_encode_ties_saturation_nan():
    enc, dec = oracle.e4m3_encode, oracle.e4m3_decode
    # 1.0 (0x38) and 1.125 (0x39): the midpoint 1.0625 goes to the even code
    assert enc(1.0625) == 0x38
    # 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 goes to 0x3A
    assert enc(1.1875) == 0x3A
    assert enc(1.0624) == 0x38 and enc(1.0626) == 0x39
    # subnormal tie: 2^-10 lies midway between 0 and 2^-9 -> 0
    assert enc(2.0 ** -10) == 0x00 and enc(1.5 * 2.0 ** -9) == 0x02
    assert enc(448.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(464.0) == 0x7E            # beyond 448: saturates, no infinity
    assert enc(np.nan) == 0x7F
    assert dec(enc(-3.3)) == -3.25


def test_e4m3_encode_matches_torch_cast():
    x = _rand(20000, scale=40.0)
    x = np.concatenate([x, _rand(2000, scale=0.01)])
    ours = oracle.e4m3_encode(x)
    # torch's cast (RNE); its saturation is applied by clamping first
    ref = torch.from_numpy(np.clip(x, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    zero = (oracle.e4m3_decode(ours) == 0) & (oracle.e4m3_decode(ref) == 0)
    assert np.all(zero | (ours == ref))


def test_dequantize_per_head_axis():
    codes = np.array([[0x38, 0x40], [0x38, 0x40]], dtype=np.uint8)  # 1.0, 2.0
    out = oracle.dequantize(codes, np.array([3.0, 5.0]), head_axis=1)
    assert np.array_equal(out, [[3.0, 10.0], [3.0, 10.0]])


# ------------------------------------------------------------------ geometry / pooling

def test_geometry_chunked():
    g = A.geometry(seqlen_q=40, seqlen_k=100, block=16)
    assert g.q_offset == 60 and g.first_qblock == 3 and g.nkb == 7
    assert g.nqb == 4                       # blocks 3,4,5,6 (positions 60..99)
    assert g.q_rows(3) == (0, 4)            # positions 60..63 -> partial block
    assert g.q_rows(6) == (36, 40)          # positions 96..99 -> ragged tail
    assert g.k_rows(6) == (96, 100)


@pytest.mark.parametrize("Sq,Sk", [(37, 37), (21, 53), (16, 48)])
def test_pool_matches_loops(Sq, Sk):
    Hq, Hkv, d, b = 6, 2, 5, 8
    G = Hq // Hkv
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    qbar, kbar, vbar, n_k = A.pool(q, k, v, Hkv, b)
    P = Sk - Sq
    first = P // b
    for h in range(Hkv):
        for il in range(qbar.shape[1]):
            i = first + il
            acc = np.zeros(d)
            n = 0
            for r in range(Sq):
                if (P + r) // b == i:
                    for g in range(G):
                        acc += q[r, h * G + g]
                        n += 1
            assert np.allclose(qbar[h, il], acc / n, rtol=0, atol=1e-13)
        for j in range(kbar.shape[1]):
            ks = [c for c in range(Sk) if c // b == j]
            assert n_k[j] == len(ks)
            assert np.allclose(kbar[h, j], sum(k[c, h] for c in ks) / len(ks), atol=1e-13)
            assert np.allclose(vbar[h, j], sum(v[c, h] for c in ks) / len(ks), atol=1e-13)


def test_pool_constant_block_is_constant():
    Sq = Sk = 32
    q = np.ones((Sq, 4, 3)) * 2.5
    k = np.repeat(np.arange(Sk, dtype=float)[:, None, None] // 8, 3, axis=2).repeat(2, axis=1)
    qbar, kbar, vbar, _ = A.pool(q, k, k, 2, 8)
    assert np.all(qbar == 2.5)
    for j in range(4):
        assert np.all(kbar[:, j] == j) and np.all(vbar[:, j] == j)


# ------------------------------------------------------------------ scores / select

def _brute_select(qbar, kbar, ids, tau):
    H, nq, _ = qbar.shape
    nk = kbar.shape[1]
    kept = np.zeros((H, nq, nk), dtype=bool)
    for h in range(H):
        for il, i in enumerate(ids):
            s = [sum(qbar[h, il, t] * kbar[h, j, t] for t in range(qbar.shape[2]))
                 for j in range(i + 1)]
            m = max(s)
            for j in range(i + 1):
                kept[h, il, j] = (s[j] >= m - tau) or j == 0 or j == i
    return kept


@pytest.mark.parametrize("tau", [0.0, 0.3, 1.0, 5.0])
def test_select_matches_loops(tau):
    qbar, kbar = _rand(2, 9, 4), _rand(2, 12, 4)
    ids = np.arange(3, 12)
    S = A.block_scores(qbar, kbar, ids)
    kept, thr = A.select(S, ids, tau)
    assert np.array_equal(kept, _brute_select(qbar, kbar, ids, tau))
    assert np.all(np.isnan(S[:, 0, 4:]))    # blocks above the diagonal are invisible


def test_select_invariants():
    qbar, kbar = _rand(3, 20, 6), _rand(3, 20, 6)
    ids = np.arange(20)
    S = A.block_scores(qbar, kbar, ids)
    prev = None
    for tau in [0.0, 0.1, 0.5, 1.0, 2.0, 4.0, np.inf]:
        kept, _ = A.select(S, ids, tau)
        assert kept[:, :, 0].all()                               # sink
        assert kept[:, ids, ids].all()                           # diagonal
        assert not kept[:, np.arange(20)[:, None] < np.arange(20)[None, :]].any()
        if prev is not None:
            assert np.all(kept >= prev)                          # monotone in tau
        prev = kept
    assert A.sparsity(prev, ids) == 0.0                          # tau = inf keeps all
    kept0, _ = A.select(S, ids, 0.0)
    for h in range(3):
        for i in range(20):
            s = S[h, i, : i + 1]
            expect = set(np.flatnonzero(s == s.max())) | {0, i}
            assert set(np.flatnonzero(kept0[h, i])) == expect    # tau = 0


def _brute_union(q, k, Hkv, b, tau):
    """Per-query-head selection united over each group, with explicit loops:
    head hq pools its own rows of each query block and applies the rule."""
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    G = Hq // Hkv
    P = Sk - Sq
    first, last = P // b, (Sk - 1) // b
    nkb = -(-Sk // b)
    kept = np.zeros((Hkv, last - first + 1, nkb), dtype=bool)
    for hq in range(Hq):
        h = hq // G
        for il, i in enumerate(range(first, last + 1)):
            rows = [r for r in range(Sq) if (P + r) // b == i]
            qm = [sum(q[r, hq, t] for r in rows) / len(rows) for t in range(d)]
            s = []
            for j in range(i + 1):
                keys = [c for c in range(Sk) if c // b == j]
                km = [sum(k[c, h, t] for c in keys) / len(keys) for t in range(d)]
                s.append(sum(qm[t] * km[t] for t in range(d)))
            m = max(s)
            for j in range(i + 1):
                if s[j] >= m - tau or j == 0 or j == i:
                    kept[h, il, j] = True
    return kept


@pytest.mark.parametrize("tau", [0.0, 0.4, 2.0])
def test_select_union_matches_loops(tau):
    Sq, Sk, Hq, Hkv, d, b = 21, 37, 6, 2, 3, 4
    q, k = _rand(Sq, Hq, d), _rand(Sk, Hkv, d)
    geo = A.geometry(Sq, Sk, b)
    qh = A.pool_q_heads(q, Sk, b)
    _, kbar, _, _ = A.pool(q, k, k, Hkv, b)
    kept, S, thr = A.select_union(qh, kbar, geo.q_block_ids(), tau)
    assert np.array_equal(kept, _brute_union(q, k, Hkv, b, tau))
    assert S.shape == (Hq, geo.nqb, geo.nkb) and thr.shape == (Hq, geo.nqb)


def test_select_union_reductions():
    Sq = Sk = 48
    Hkv, d, b = 2, 5, 8
    k = _rand(Sk, Hkv, d)
    ids = A.geometry(Sq, Sk, b).q_block_ids()
    # one head per group: the union is the group-mean selection
    q1 = _rand(Sq, Hkv, d)
    _, kbar, _, _ = A.pool(q1, k, k, Hkv, b)
    qbar, _, _, _ = A.pool(q1, k, k, Hkv, b)
    for tau in [0.0, 0.5, 3.0]:
        ku, _, _ = A.select_union(A.pool_q_heads(q1, Sk, b), kbar, ids, tau)
        km, _ = A.select(A.block_scores(qbar, kbar, ids), ids, tau)
        assert np.array_equal(ku, km)
    # heads of a group with identical queries: the union is again the group-mean selection
    G = 3
    qg = np.repeat(_rand(Sq, Hkv, 1, d), G, axis=2).reshape(Sq, Hkv * G, d)
    qbar, _, _, _ = A.pool(qg, k, k, Hkv, b)
    for tau in [0.0, 0.5, 3.0]:
        ku, _, _ = A.select_union(A.pool_q_heads(qg, Sk, b), kbar, ids, tau)
        km, _ = A.select(A.block_scores(qbar, kbar, ids), ids, tau)
        assert np.array_equal(ku, km)
    # the union contains every head's own selection, the sink and the diagonal; tau = inf keeps all
    q = _rand(Sq, Hkv * G, d)
    qh = A.pool_q_heads(q, Sk, b)
    ku, S, thr = A.select_union(qh, kbar, ids, 0.7)
    kh, _ = A.select(S, ids, 0.7)
    assert np.all(ku >= kh.reshape(Hkv, G, *kh.shape[1:]).any(axis=1))
    assert ku[:, :, 0].all() and ku[:, np.arange(len(ids)), ids].all()
    ki, _, _ = A.select_union(qh, kbar, ids, np.inf)
    assert A.sparsity(ki, ids) == 0.0


def _brute_head_max(q, k, Hkv, b, tau):
    """Group score = the largest per-head score, with explicit loops: head hq
    pools its own rows of each query block; the group keeps block j when that
    maximum is within tau of the row's largest maximum."""
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    G = Hq // Hkv
    P = Sk - Sq
    first, last = P // b, (Sk - 1) // b
    nkb = -(-Sk // b)
    kept = np.zeros((Hkv, last - first + 1, nkb), dtype=bool)
    for h in range(Hkv):
        for il, i in enumerate(range(first, last + 1)):
            rows = [r for r in range(Sq) if (P + r) // b == i]
            s = []
            for j in range(i + 1):
                keys = [c for c in range(Sk) if c // b == j]
                km = [sum(k[c, h, t] for c in keys) / len(keys) for t in range(d)]
                best = -np.inf
                for hq in range(h * G, (h + 1) * G):
                    qm = [sum(q[r, hq, t] for r in rows) / len(rows) for t in range(d)]
                    best = max(best, sum(qm[t] * km[t] for t in range(d)))
                s.append(best)
            m = max(s)
            for j in range(i + 1):
                if s[j] >= m - tau or j == 0 or j == i:
                    kept[h, il, j] = True
    return kept


@pytest.mark.parametrize("tau", [0.0, 0.4, 2.0])
def test_select_head_max_matches_loops(tau):
    Sq, Sk, Hq, Hkv, d, b = 21, 37, 6, 2, 3, 4
    q, k = _rand(Sq, Hq, d), _rand(Sk, Hkv, d)
    geo = A.geometry(Sq, Sk, b)
    qh = A.pool_q_heads(q, Sk, b)
    _, kbar, _, _ = A.pool(q, k, k, Hkv, b)
    kept, S, thr = A.select_head_max(qh, kbar, geo.q_block_ids(), tau)
    assert np.array_equal(kept, _brute_head_max(q, k, Hkv, b, tau))
    assert S.shape == (Hkv, geo.nqb, geo.nkb) and thr.shape == (Hkv, geo.nqb)
    if tau == 0.4:
        # the case tells the variants apart: a max that averaged or united instead would fail
        ku, _, _ = A.select_union(qh, kbar, geo.q_block_ids(), tau)
        qbar, _, _, _ = A.pool(q, k, k, Hkv, b)
        km, _ = A.select(A.block_scores(qbar, kbar, geo.q_block_ids()), geo.q_block_ids(), tau)
        assert not np.array_equal(kept, ku) and not np.array_equal(kept, km)


def test_select_head_max_hand_case():
    """One KV head, two query heads with pooled queries (1, 0) and (0, 1),
    key-block means (0,0), (1,1), (3,-3), (-5,-5); row i = 3, tau = 1.5.
    Per-head scores: head 0 [0, 1, 3, -5], head 1 [0, 1, -3, -5].
    max: [0, 1, 3, -5], threshold 1.5, keeps {2} + sink + diagonal.
    mean (qbar (0.5, 0.5)): [0, 1, 0, -5], threshold -0.5, keeps {0, 1, 2, 3}.
    union: head 0 keeps {2}, head 1 (threshold -0.5) keeps {0, 1}: {0, 1, 2, 3}."""
    ids = np.arange(4)
    kbar = np.array([[[0.0, 0.0], [1.0, 1.0], [3.0, -3.0], [-5.0, -5.0]]])
    qh = np.zeros((2, 4, 2))
    qh[0, :, 0] = 1.0
    qh[1, :, 1] = 1.0
    kept, S, thr = A.select_head_max(qh, kbar, ids, 1.5)
    assert np.array_equal(S[0, 3], [0.0, 1.0, 3.0, -5.0]) and thr[0, 3] == 1.5
    assert set(np.flatnonzero(kept[0, 3])) == {0, 2, 3}
    ku, _, _ = A.select_union(qh, kbar, ids, 1.5)
    km, _ = A.select(A.block_scores(qh.mean(axis=0, keepdims=True), kbar, ids), ids, 1.5)
    assert set(np.flatnonzero(ku[0, 3])) == {0, 1, 2, 3} == set(np.flatnonzero(km[0, 3]))
    # row 1 (blocks 0, 1): both kept as sink and diagonal
    assert set(np.flatnonzero(kept[0, 1])) == {0, 1} and not kept[0, 1, 2:].any()


def test_select_head_max_reductions():
    Sq = Sk = 48
    Hkv, d, b = 2, 5, 8
    k = _rand(Sk, Hkv, d)
    ids = A.geometry(Sq, Sk, b).q_block_ids()
    # one head per group, or identical heads: the maximum is the group-mean selection
    q1 = _rand(Sq, Hkv, d)
    G = 3
    qg = np.repeat(_rand(Sq, Hkv, 1, d), G, axis=2).reshape(Sq, Hkv * G, d)
    for q in (q1, qg):
        qbar, kbar, _, _ = A.pool(q, k, k, Hkv, b)
        for tau in [0.0, 0.5, 3.0]:
            kx, Sx, _ = A.select_head_max(A.pool_q_heads(q, Sk, b), kbar, ids, tau)
            Sm = A.block_scores(qbar, kbar, ids)
            km, _ = A.select(Sm, ids, tau)
            assert np.array_equal(kx, km)
            np.testing.assert_allclose(Sx, Sm, rtol=1e-12, atol=1e-12)
    # tau = inf keeps all; sink and diagonal always kept
    q = _rand(Sq, Hkv * G, d)
    _, kbar, _, _ = A.pool(q, k, k, Hkv, b)
    kx, _, _ = A.select_head_max(A.pool_q_heads(q, Sk, b), kbar, ids, -1.0)
    assert kx[:, :, 0].all() and kx[:, np.arange(len(ids)), ids].all()
    ki, _, _ = A.select_head_max(A.pool_q_heads(q, Sk, b), kbar, ids, np.inf)
    assert A.sparsity(ki, ids) == 0.0


def test_score_band_mask_hand_cases():
    """The band is |S - thr| <= band per (head, row), NaN (invisible) entries
    outside it.  Values are exact binary fractions, so the <= edge is exact;
    the two heads and two rows have different thresholds, so a transposed or
    mis-broadcast threshold fails."""
    t = 2.0 ** -10                                   # 0.0009765625 < 1e-3 < 2^-9
    S = np.array([[[0.5, 0.5 + t, 0.5 - t, 0.5 + 2 * t],      # head 0, row 0: thr 0.5
                   [1.0, 0.25, 0.25 - t, np.nan]],            # head 0, row 1: thr 0.25
                  [[-1.0, -1.0 - t, 0.5, -1.0 + 4 * t],       # head 1, row 0: thr -1
                   [3.0, 3.0 + t, 2.0, np.nan]]])             # head 1, row 1: thr 3
    thr = np.array([[0.5, 0.25], [-1.0, 3.0]])
    want = np.array([[[True, True, True, False],
                      [False, True, True, False]],
                     [[True, True, False, False],
                      [True, True, False, False]]])
    assert np.array_equal(A.score_band_mask(S, thr), want)
    # a wider band takes in the 2t and 4t entries, never the NaN ones
    want2 = want.copy()
    want2[0, 0, 3] = want2[1, 0, 3] = True
    assert np.array_equal(A.score_band_mask(S, thr, band=4 * t), want2)
    # band 0: exactly the entries equal to their threshold
    assert np.array_equal(A.score_band_mask(S, thr, band=0.0), S == thr[:, :, None])


def test_union_band_mask_hand_cases():
    """A group's block is in the band when ANY query head of the group
    (heads h*G .. h*G+G-1) scores it within the band of that head's own
    threshold.  Four query heads, two groups: the in-band entries are placed
    so that grouping heads by hq % Hkv instead of hq // G, or using another
    head's threshold, gives a different answer."""
    t = 2.0 ** -10
    Hq, Hkv, nqb, nkb = 4, 2, 1, 4
    thr = np.array([[0.0], [1.0], [2.0], [3.0]])     # per query head, one row
    S = np.full((Hq, nqb, nkb), 10.0)                # far from every threshold
    S[0, 0, 0] = 0.0 + t                             # head 0 (group 0) in band at block 0
    S[1, 0, 1] = 1.0 - t                             # head 1 (group 0) in band at block 1
    S[2, 0, 2] = 2.0                                 # head 2 (group 1) in band at block 2
    S[3, 0, 3] = 0.0                                 # head 3: within band of head 0's threshold only
    S[3, 0, 1] = np.nan                              # invisible entry: never in band
    want = np.zeros((Hkv, nqb, nkb), dtype=bool)
    want[0, 0, [0, 1]] = True
    want[1, 0, 2] = True
    got = A.union_band_mask(S, thr, Hkv)
    assert got.shape == (Hkv, nqb, nkb)
    assert np.array_equal(got, want)
    # explicit loop over groups and heads
    loop = np.zeros_like(want)
    G = Hq // Hkv
    for h in range(Hkv):
        for g in range(G):
            hq = h * G + g
            for j in range(nkb):
                x = S[hq, 0, j]
                if not np.isnan(x) and abs(x - thr[hq, 0]) <= 1e-3:
                    loop[h, 0, j] = True
    assert np.array_equal(got, loop)


def test_sparsity_definition():
    kept = np.zeros((1, 4, 4), dtype=bool)
    kept[0, np.arange(4), np.arange(4)] = True    # 4 kept of 1+2+3+4 = 10 visible
    assert A.sparsity(kept, np.arange(4)) == pytest.approx(0.6)


# ------------------------------------------------------------------ attention

def _naive_attention(q, k, v, Hkv, scale, key_ok=None):
    """Textbook causal softmax attention, one query row and one key at a time.
    key_ok(hq, r, c) restricts the keys (block sparsity without correction)."""
    Sq, Hq, d = q.shape
    Sk = k.shape[0]
    G = Hq // Hkv
    P = Sk - Sq
    O = np.zeros((Sq, Hq, d))
    L = np.zeros((Hq, Sq))
    for hq in range(Hq):
        h = hq // G
        for r in range(Sq):
            logits = []
            vals = []
            for c in range(P + r + 1):
                if key_ok is None or key_ok(hq, r, c):
                    logits.append(scale * sum(q[r, hq, t] * k[c, h, t] for t in range(d)))
                    vals.append(v[c, h])
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            s = sum(w)
            O[r, hq] = sum(wi * vi for wi, vi in zip(w, vals)) / s
            L[hq, r] = m + math.log(s)
    return O, L


@pytest.mark.parametrize("Sq,Sk", [(40, 40), (19, 45)])
def test_all_kept_equals_textbook_dense(Sq, Sk):
    Hq, Hkv, d, b = 4, 2, 6, 8
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    scale = 1 / math.sqrt(d)
    O0, L0 = _naive_attention(q, k, v, Hkv, scale)
    res = A.sparse_prefill(q, k, v, Hkv, b, tau=np.inf)
    assert np.abs(res["O"] - O0).max() < 1e-12
    assert np.abs(res["LSE"] - L0).max() < 1e-12
    Od, Ld = A.dense_attention(q, k, v, Hkv, scale)
    assert np.abs(Od - O0).max() < 1e-12 and np.abs(Ld - L0).max() < 1e-12


def test_sparse_without_correction_equals_masked_textbook():
    Sq = Sk = 48
    Hq, Hkv, d, b = 4, 2, 6, 8
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    res = A.sparse_prefill(q, k, v, Hkv, b, tau=0.2, mean_correction=False)
    kept = res["kept"]
    assert A.sparsity(kept, res["geo"].q_block_ids()) > 0.2
    G = Hq // Hkv
    ok = lambda hq, r, c: kept[hq // G, r // b, c // b]
    O0, L0 = _naive_attention(q, k, v, Hkv, res["scale"], ok)
    assert np.abs(res["O"] - O0).max() < 1e-12
    assert np.abs(res["LSE"] - L0).max() < 1e-12


@pytest.mark.parametrize("tau", [0.0, 0.05, 0.5])
def test_mean_correction_exact_for_identical_keys(tau):
    """Keys identical within each block: the pseudo-key (logit + ln n_j, value
    vbar_j) carries exactly the mass and value of the dropped block, so the
    corrected sparse output equals dense attention."""
    Sq = Sk = 64
    Hq, Hkv, d, b = 4, 2, 8, 8
    kb = _rand(Sk // b, Hkv, d, scale=2.0)
    k = np.repeat(kb, b, axis=0)
    q, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d)
    res = A.sparse_prefill(q, k, v, Hkv, b, tau=tau, mean_correction=True)
    assert A.sparsity(res["kept"], res["geo"].q_block_ids()) > 0.3
    Od, Ld = A.dense_attention(q, k, v, Hkv, res["scale"])
    assert np.abs(res["O"] - Od).max() < 1e-12
    assert np.abs(res["LSE"] - Ld).max() < 1e-12
    off = A.sparse_prefill(q, k, v, Hkv, b, tau=tau, mean_correction=False)
    assert np.abs(off["O"] - Od).max() > 1e-3          # the correction mattered


def test_constant_values_give_constant_output():
    Sq, Sk = 30, 70
    Hq, Hkv, d, b = 4, 1, 5, 8
    q, k = _rand(Sq, Hq, d), _rand(Sk, Hkv, d)
    v = np.broadcast_to(np.arange(d, dtype=float), (Sk, Hkv, d)).copy()
    for corr in (True, False):
        res = A.sparse_prefill(q, k, v, Hkv, b, tau=0.1, mean_correction=corr)
        assert np.abs(res["O"] - np.arange(d)).max() < 1e-12


def test_correction_identity_with_out_v2_ingredients():
    """Fold == O_supp - mu_q * (O_supp - Vbar_drop) for every row."""
    Sq = Sk = 64
    Hq, Hkv, d, b = 4, 2, 8, 8
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    res = A.sparse_prefill(q, k, v, Hkv, b, tau=0.1)
    G = Hq // Hkv
    for i in range(1, 8):
        parts = A.correction_split(q, k, v, res["kept"], res["kbar"], res["vbar"],
                                   res["n_k"], Hkv, b, res["scale"], i)
        for h, (Os, Vd, mu) in enumerate(parts):
            fold = res["O"][i * b:(i + 1) * b, h * G:(h + 1) * G].reshape(b * G, d)
            assert np.abs(fold - (Os - mu[:, None] * (Os - Vd))).max() < 1e-12
            if not res["kept"][h, i, : i + 1].all():
                assert mu.min() > 0


def test_tau_inf_and_no_correction_agree_with_dense():
    Sq, Sk = 33, 80
    Hq, Hkv, d, b = 8, 2, 4, 16
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    Od, _ = A.dense_attention(q, k, v, Hkv, 0.5)
    for corr in (True, False):
        res = A.sparse_prefill(q, k, v, Hkv, b, tau=np.inf, scale=0.5, mean_correction=corr)
        assert np.abs(res["O"] - Od).max() < 1e-12


def test_gqa_head_mapping():
    """Query head hq must read KV head hq // G: permuting the KV heads and the
    matching query-head groups together permutes the output heads."""
    Sq = Sk = 32
    Hq, Hkv, d, b = 6, 3, 4, 8
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    res = A.sparse_prefill(q, k, v, Hkv, b, tau=0.3)
    perm = np.array([2, 0, 1])
    qperm = q.reshape(Sq, Hkv, 2, d)[:, perm].reshape(Sq, Hq, d)
    res2 = A.sparse_prefill(qperm, k[:, perm], v[:, perm], Hkv, b, tau=0.3)
    Operm = res["O"].reshape(Sq, Hkv, 2, d)[:, perm].reshape(Sq, Hq, d)
    assert np.abs(res2["O"] - Operm).max() < 1e-12
    # and the mapping is grouped (hq // G), not strided (hq % Hkv)
    G = Hq // Hkv
    ok = lambda hq, r, c: res["kept"][hq // G, r // b, c // b]
    res_nc = A.sparse_prefill(q, k, v, Hkv, b, tau=0.3, mean_correction=False)
    O0, _ = _naive_attention(q, k, v, Hkv, res["scale"], ok)
    assert np.abs(res_nc["O"] - O0).max() < 1e-12


def test_q_block_subset_matches_full():
    Sq = Sk = 64
    Hq, Hkv, d, b = 4, 2, 8, 8
    q, k, v = _rand(Sq, Hq, d), _rand(Sk, Hkv, d), _rand(Sk, Hkv, d)
    full = A.sparse_prefill(q, k, v, Hkv, b, tau=0.2)
    part = A.sparse_prefill(q, k, v, Hkv, b, tau=0.2, q_blocks=[0, 5, 7])
    for i in (0, 5, 7):
        sl = slice(i * b, (i + 1) * b)
        assert np.array_equal(part["O"][sl], full["O"][sl])
    assert np.isnan(part["O"][8:40]).all()


def test_chunked_rows_equal_full_prefill_rows():
    """Selection of a query block depends only on its own rows and the keys
    before it, so a block-aligned chunk reproduces the full prefill's rows."""
    S, C = 96, 40
    Hq, Hkv, d, b = 4, 2, 8, 8
    q, k, v = _rand(S, Hq, d), _rand(S, Hkv, d), _rand(S, Hkv, d)
    full = A.sparse_prefill(q, k, v, Hkv, b, tau=0.15)
    chunk = A.sparse_prefill(q[S - C:], k, v, Hkv, b, tau=0.15)
    assert np.abs(chunk["O"] - full["O"][S - C:]).max() < 1e-12
