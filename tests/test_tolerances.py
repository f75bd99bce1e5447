"""The numbers the fp8 tolerances rest on (CPU only).

The fp8 attention kernel stores the softmax numerators P = 2^x of each
64-key superchunk as e4m3 codes c = RNE(8 (x + 7) - 0.34), clamped to
[0, 255], after a power-of-two scale that puts the superchunk's largest x in
[7, 8): the exponent and mantissa bits of the code read as one fixed-point
number of x + 7, a log-linear approximation of 2^x with its error centred.
Its decoded value is checked here against 2^x with the e4m3 decoder of the
oracle (written from the format definition), over the range the scaled
codes use: the relative error must stay within the factor the fp8 LSE
tolerance allows, and its spread must stay close to that of exact
round-to-nearest e4m3 (the output tolerance is not changed by the code).
"""

import numpy as np

import oracle
from tests.helpers import FP8_LSE_ABS

SHIFT = 0.34  # the code's centring shift


def _codes(x):
    return np.clip(np.rint(8.0 * (x + 7.0) - SHIFT), 0, 255).astype(np.uint8)


def test_code_range_and_monotone():
    x = np.linspace(-12.0, 8.0 - 1e-9, 200001)
    c = _codes(x)
    assert c.max() <= 0x78            # the largest x of a superchunk (< 8) stays at or below 256
    assert not np.any((c & 0x7F) == 0x7F)  # never an e4m3 NaN
    assert np.all(np.diff(c.astype(np.int64)) >= 0)


def test_relative_error_within_lse_tolerance():
    # normal range of the codes (values 2^-6 .. 256), fine grid
    x = np.linspace(-6.0, 8.0 - 1e-9, 1400001)
    r = oracle.e4m3_decode(_codes(x)) / 2.0 ** x
    lr = np.log(r)
    assert np.abs(lr).max() < 0.0730
    assert np.abs(lr).max() < FP8_LSE_ABS
    # spread: within 25% of round-to-nearest e4m3's (std of ln r 0.0265)
    assert lr.std() < 1.25 * 0.0265
    # centred: the mean ratio is within 1.2% of 1
    assert abs(r.mean() - 1.0) < 0.012


def test_subnormal_and_underflow_codes_are_small():
    # below the normal range the codes only ever underestimate by at most
    # the smallest normal value, 2^-6, relative to a superchunk maximum >= 128
    x = np.linspace(-30.0, -6.0, 100001)
    v = oracle.e4m3_decode(_codes(x))
    assert np.all(v <= 2.0 ** -6 + 1e-12)
    assert np.all(np.abs(v - 2.0 ** x) <= 2.0 ** -6)


def test_unorm16_route_gives_the_rounded_code():
    # The kernel forms y = (256 c + 127.5) / 65535 with one fp32 FMA per
    # score, converts two scores at a time to unorm16 (clamp to [0, 1], then
    # round(65535 y)) and keeps the high byte of each.  That byte is the code
    # c rounded to nearest and clamped to [0, 255]: exactly, away from the
    # half-integers; within 1/256 of one, a convert that truncated instead of
    # rounding would move the code by one step (the same error as a shift of
    # the centring constant by 1/512).
    c = np.linspace(-3.0, 124.0, 2_000_001)
    y = ((256.0 * c + 127.5) / 65535.0).astype(np.float32)
    u = np.clip(y.astype(np.float64), 0.0, 1.0) * 65535.0
    hi_rne = (np.rint(u) // 256).astype(np.int64)
    hi_trunc = (np.floor(u) // 256).astype(np.int64)
    want = np.clip(np.rint(c), 0, 255).astype(np.int64)
    frac = c - np.floor(c)
    away = np.abs(frac - 0.5) > 1e-5
    assert np.array_equal(hi_rne[away], want[away])
    assert np.abs(hi_trunc - want).max() <= 1
    assert np.all(np.abs(frac[hi_trunc != want] - 0.5) <= 1.0 / 256)
    # the four high bytes gathered by the byte permute (selector 0x07050301
    # over the pair words lo = (y0, y1), hi = (y2, y3)) are y0, y1, y2, y3 in
    # byte order 0-3 of the P register
    lo = np.uint32(0x12AB) | (np.uint32(0x34CD) << np.uint32(16))
    hi = np.uint32(0x56EF) | (np.uint32(0x7801) << np.uint32(16))
    src = [(int(lo) >> (8 * k)) & 0xFF for k in range(4)] + [(int(hi) >> (8 * k)) & 0xFF for k in range(4)]
    sel = 0x07050301
    word = sum(src[(sel >> (8 * k)) & 0xFF] << (8 * k) for k in range(4))
    assert word == 0x78563412
