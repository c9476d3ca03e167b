"""Storage number formats used by the latent cache, written from their
definitions (oracle; test infrastructure only).

bf16: 8 significant bits, fp32 exponent range, round-to-nearest-even.
e4m3fn (OCP 8-bit float, "fn" = finite, no infinities): sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal with value
2^-6 * m/8; codes 0x7F/0xFF are NaN; largest finite magnitude 448.

The pages only say the deployed cache is quantised to about 6 bits per
element on average (DeepSeek-V2 reading card, "Method adaptation", serving
paragraph; discosf explainer, throughput paragraph) without naming a format;
the 8-bit e4m3fn format with one fp32 scale per token is the plain stand-in
taken here.
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
