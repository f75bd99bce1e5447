"""FP8 E4M3 decoding for the oracle (test infrastructure only).

[EXP] §2.3 names FP8 E4M3 inputs with scale calibration; [ABS] says the
operator supports FP8 inference.  The pages do not spell out the bit layout.
Reading taken: the OCP 8-bit floating point E4M3 format ("e4m3fn"):

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 encodes subnormals  (-1)^s * (m/8) * 2^-6;
* exponent fields 1..15 encode normals (-1)^s * (1 + m/8) * 2^(e-7),
  except S.1111.111, the only NaN encoding; there are no infinities;
* largest finite magnitude 0x7E = 448, smallest subnormal 2^-9.

Values are dequantized as  code_value * scale  with one fp32 scale per head
(the workload's per-head calibration; a per-tensor scale is the special case
of equal scales).

Encoding (for an e4m3 output, [EXP] §2.3: FP8 input and output): a value
x / scale is rounded to the nearest finite E4M3 value, ties to the code with
an even mantissa (round-to-nearest-even), and magnitudes beyond 448 saturate
to +-448 (e4m3fn has no infinity to overflow into).
"""

import numpy as np


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64, straight from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = (man / 8.0) * 2.0 ** -6
    nor = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    val = np.where(exp == 0, sub, nor) * sign
    val = np.where((exp == 0xF) & (man == 0x7), np.nan, val)
    return val


def _finite_table():
    """The 127 non-negative finite magnitudes, codes 0x00 .. 0x7E, ascending."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, e4m3_decode(codes)


def e4m3_encode(x):
    """float64 values -> uint8 E4M3 codes: nearest finite value, ties to even
    mantissa, saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    codes, mags = _finite_table()
    a = np.minimum(np.abs(x), mags[-1])
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)  # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    mag_code = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = np.where(np.signbit(x) & (mag_code != 0), 0x80, 0x00).astype(np.uint8)
    out = mag_code | sign
    return np.where(np.isnan(x), np.uint8(0x7F), out).astype(np.uint8)


def dequantize(codes, scale, head_axis):
    """codes (uint8, any shape) * per-head scale broadcast along ``head_axis``."""
    vals = e4m3_decode(codes)
    s = np.asarray(scale, dtype=np.float64)
    shape = [1] * vals.ndim
    shape[head_axis] = s.shape[0]
    return vals * s.reshape(shape)
