"""OCP 8-bit E4M3 ("E4M3FN") codec in float64 (oracle; test infrastructure).

The 8-bit path of [FlashInfer-Sage] (code §1, the README formula) stores P as
an E4M3 value of 448·p; 448 is the largest finite E4M3 number of the OCP
8-bit floating point format, which this codec follows, written from the
public OCP FP8 definition:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 1..15: value 2^(e-7) · (1 + m/8); exponent field 0:
  subnormal 2^-6 · m/8 (smallest 2^-9);
* no infinities; S.1111.111 is NaN, so the largest finite value is
  2^8 · 1.75 = 448;
* rounding to nearest, ties to even; finite values beyond 448 saturate to
  ±448 (448·p never exceeds 448 for p ≤ 1).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3 byte codes (uint8), RNE, saturating."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    sign = np.signbit(x)
    a = np.where(nan, 0.0, np.abs(x))
    _, ex = np.frexp(a)  # a = f * 2^ex with f in [0.5, 1)
    e = np.maximum(ex - 1, _MIN_NORMAL_EXP)  # a in [2^e, 2^(e+1)) for normals
    quantum = np.ldexp(1.0, e - 3)  # spacing of E4M3 values in that binade
    r = np.rint(a / quantum) * quantum  # exact power-of-two scaling; rint = ties-to-even
    r = np.minimum(r, E4M3_MAX)
    # encode the (now representable) magnitude r
    sub = r < 2.0 ** _MIN_NORMAL_EXP
    m_sub = np.rint(r / 2.0 ** -9).astype(np.int64)  # 0..7 (8 would be normal)
    _, ex_r = np.frexp(np.where(sub, 1.0, r))
    e_r = ex_r - 1
    m_norm = np.rint((np.where(sub, 1.0, r) / np.ldexp(1.0, e_r) - 1.0) * 8).astype(np.int64)
    code = np.where(sub, m_sub, ((e_r + 7) << 3) | m_norm)
    code = code | (sign.astype(np.int64) << 7)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Exact float64 value of E4M3 byte codes (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val
