"""Storage number formats used by the latent cache, written from their
definitions (oracle; test infrastructure only).

bf16: 8 significant bits, fp32 exponent range, round-to-nearest-even.
e4m3fn (OCP 8-bit float, "fn" = finite, no infinities): sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal with value
2^-6 * m/8; codes 0x7F/0xFF are NaN; largest finite magnitude 448.

e2m3 (OCP 6-bit float "FP6 E2M3"): sign bit, 2 exponent bits with bias 1, 3
mantissa bits; exponent field 0 is subnormal with value m/8; no infinities or
NaN; largest magnitude 7.5. e8m0: an 8-bit biased exponent, value 2^(code-127).

The pages only say the deployed cache is quantised to about 6 bits per
element on average (DeepSeek-V2 reading card, "Method adaptation", serving
paragraph; discosf explainer, throughput paragraph) without naming a format.
Two stand-ins are taken: the 8-bit e4m3fn format with one fp32 scale per
token, and the ~6-bit one: e2m3 elements in blocks of 32 along the row with
one e8m0 scale per block (6.25 bits per element), the OCP microscaling layout.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned
    as fp64. Subnormal bf16 values (below 2^-126) keep a 2^-133 quantum."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| = m * 2^e with 0.5 <= m < 1
    e = np.maximum(e, -125)                 # below 2^-126 the quantum stops shrinking
    quantum = np.ldexp(1.0, e - 8)          # 8 significant bits
    with np.errstate(invalid="ignore"):
        return np.where(x == 0, x, np.round(x / quantum) * quantum)


def round_f32(x) -> np.ndarray:
    """Round fp64 values to fp32 (IEEE round-to-nearest-even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each uint8 e4m3fn code, as fp64 (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    sub = np.ldexp(man / 8.0, -6)
    val = sign * np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_value_table() -> np.ndarray:
    """The 127 non-negative finite e4m3fn values in code order 0x00..0x7E."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Round fp64 values to e4m3fn codes: round-to-nearest-even on the
    3-bit mantissa, magnitudes above 448 saturate to 448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                      # ax = m * 2^e, 0.5 <= m < 1
    e = np.maximum(e, -5)                    # below 2^-6 the quantum is 2^-9
    quantum = np.ldexp(1.0, e - 4)           # 4 significant bits
    with np.errstate(invalid="ignore", over="ignore"):
        mag = np.round(ax / quantum) * quantum
    mag = np.minimum(mag, E4M3_MAX)
    table = e4m3_value_table()
    idx = np.searchsorted(table, np.nan_to_num(mag, nan=0.0))
    idx = np.clip(idx, 0, 0x7E)
    assert np.all((table[idx] == mag) | np.isnan(x)), "encode produced a non-code value"
    code = idx.astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code)   # sign kept, also for zero
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


E2M3_MAX = 7.5
MX_BLOCK = 32


def e2m3_decode(codes) -> np.ndarray:
    """Value of each 6-bit e2m3 code (0..63), as fp64."""
    c = np.asarray(codes, dtype=np.int64)
    if np.any((c < 0) | (c > 63)):
        raise ValueError("e2m3 codes are 6-bit")
    sign = np.where(c & 0x20, -1.0, 1.0)
    exp = (c >> 3) & 0x3
    man = (c & 0x7).astype(np.float64)
    return sign * np.where(exp == 0, man / 8.0, np.ldexp(1.0 + man / 8.0, exp - 1))


def e2m3_value_table() -> np.ndarray:
    """The 32 non-negative e2m3 values in code order 0..31 (increasing)."""
    return e2m3_decode(np.arange(32))


def e2m3_encode(x) -> np.ndarray:
    """Round fp64 values to e2m3 codes: round to nearest, ties to the even
    code (even mantissa), magnitudes above 7.5 saturate to 7.5; the sign is
    kept, also for zero."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("e2m3 has no NaN")
    ax = np.abs(x)
    table = e2m3_value_table()
    hi = np.clip(np.searchsorted(table, ax), 0, 31)      # first value >= ax
    lo = np.clip(hi - 1, 0, 31)
    d_lo, d_hi = ax - table[lo], table[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(ax >= E2M3_MAX, 31, np.where(pick_hi, hi, lo))
    return np.where(np.signbit(x), code | 0x20, code).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent of an e2m3 block with largest magnitude amax:
    floor(log2(amax)) - 2 (2 = e2m3's largest exponent), so amax / 2^X lies in
    [4, 8); clamped to e8m0's [-127, 127]; an all-zero block takes -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))       # amax = m 2^e, 0.5 <= m < 1
    x = np.where(amax > 0, e - 1 - 2, -127)
    return np.clip(x, -127, 127).astype(np.int64)


def pack6(codes) -> np.ndarray:
    """Pack 6-bit codes [n, k] (k a multiple of 4) little-endian: code i takes
    bits 6i .. 6i+5 of the row's bit string; returns uint8 [n, 3k/4]."""
    c = np.asarray(codes, dtype=np.int64)
    n, k = c.shape
    g = c.reshape(n, k // 4, 4)
    word = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)   # 24 bits
    out = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
    return out.reshape(n, 3 * k // 4).astype(np.uint8)


def unpack6(packed) -> np.ndarray:
    """Inverse of pack6: uint8 [n, 3k/4] -> codes [n, k]."""
    b = np.asarray(packed, dtype=np.int64)
    n, m = b.shape
    t = b.reshape(n, m // 3, 3)
    word = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)
    out = np.stack([word & 63, (word >> 6) & 63, (word >> 12) & 63, (word >> 18) & 63], axis=-1)
    return out.reshape(n, 4 * m // 3)
