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


def dequantize(codes, scale, head_axis):
    """codes (uint8, any shape) * per-head scale broadcast along ``head_axis``."""
    vals = e4m3_decode(codes)
    s = np.asarray(scale, dtype=np.float64)
    shape = [1] * vals.ndim
    shape[head_axis] = s.shape[0]
    return vals * s.reshape(shape)
