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
