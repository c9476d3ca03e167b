"""fp64 oracle of MLA append and decode (test infrastructure only).

Sources (the pages print no equations; each step cites the passage it rests on):
  [A] discosf explainer, "long-context bottleneck" section: MHA caches
      2*n_h*d_h*l elements per token; MLA compresses each token's hidden state
      to a latent c_KV with d_c = 512, caches only that, and recovers K/V by
      up-projection at attention time; W_UK can be folded into W_Q and W_UV
      into W_O; the cache equals GQA with 2.25 groups.
  [B] discosf explainer, "decoupled RoPE and YaRN" section: RoPE cannot act on
      the compressed key without breaking the absorption, so an extra
      decoupled query/key pair of width d_Rh = 64 per head carries RoPE; the
      cache grows by d_Rh*l only, i.e. the RoPE key is shared by all heads.
  [C] DeepSeek-V2 reading card, "Bottlenecks" and "Method adaptation": MLA
      caches (d_c + d_h^R)*l elements; d_c + d_h^R = 576; 60 layers, 128K
      context and 6-bit elements give about 3.4 GB at batch 1 and about 217 GB
      at batch 64.

Readings taken where the pages are silent (each listed in the design notes):
  R1  the RoPE part enters the score by concatenation:
      score = q_nope.k_nope + q_pe.k_pe, scaled by 1/sqrt(128 + 64);
  R2  k_pe is one 64-vector per token shared by all heads [B]; q_pe is per head;
  R3  RoPE rotates interleaved pairs (2i, 2i+1) by angle pos*theta_i with
      theta_i = base^(-2i/64), angles formed in fp64; pos is the 0-based slot
      of the token inside its sequence; decode applies no RoPE (q_pe arrives
      rotated);
  R4  a query attends all L_b cached rows of its sequence (no mask); L_b >= 1;
  R5  W_UK[h] is [128 x 512] with k = W_UK[h] c; W_UV[h] is [512 x 128] with
      v = W_UV[h]^T c; both have fan-in 512 at initialisation;
  R6  no normalisation of c_KV; c_KV = W_DKV h, k = W_KR h;
  R7  fp8 cache: e4m3fn codes with one fp32 scale per token,
      scale = fp32(max|row| / 448) (1 for an all-zero row),
      code = round-to-nearest-even, saturating, of row / scale.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .numerics import round_bf16, round_f32, e4m3_decode, e4m3_encode, E4M3_MAX

D_C = 512
D_R = 64
D_ROW = D_C + D_R
D_NOPE = 128
D_V = 128


def softmax_scale() -> float:
    """1/sqrt(d_nope + d_R): the score is a dot product over 128 + 64 dims (R1)."""
    return 1.0 / np.sqrt(D_NOPE + D_R)


# ----------------------------------------------------------------------------
# cache-size closed forms ([A], [C])
# ----------------------------------------------------------------------------
def mla_cache_elements_per_token(d_c: int = D_C, d_r: int = D_R, layers: int = 1) -> int:
    """(d_c + d_h^R) * l elements per token [C]."""
    return (d_c + d_r) * layers


def mha_cache_elements_per_token(n_h: int, d_h: int, layers: int = 1) -> int:
    """2 * n_h * d_h * l elements per token for standard multi-head attention [A]."""
    return 2 * n_h * d_h * layers


def gqa_equivalent_groups(d_h: int, d_c: int = D_C, d_r: int = D_R) -> float:
    """Number of GQA groups g whose cache 2*g*d_h equals the MLA cache [A]."""
    return (d_c + d_r) / (2.0 * d_h)


def cache_bytes(tokens: int, layers: int, bits_per_element: float, batch: int = 1,
                d_c: int = D_C, d_r: int = D_R) -> float:
    """Bytes of MLA cache for `batch` sequences of `tokens` tokens [C]."""
    return mla_cache_elements_per_token(d_c, d_r, layers) * tokens * batch * bits_per_element / 8.0


# ----------------------------------------------------------------------------
# decoupled RoPE ([B], reading R3)
# ----------------------------------------------------------------------------
def rope_inv_freq(base: float, d_r: int = D_R) -> np.ndarray:
    """theta_i = base^(-2i/d_r), i = 0 .. d_r/2-1, in fp64."""
    i = np.arange(d_r // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d_r)


def rope_rotate(k: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each interleaved pair (k[2i], k[2i+1]) of the last axis by
    pos * theta_i. `k` is [..., 64], `pos` broadcasts against k[..., 0]."""
    k = np.asarray(k, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    phi = pos * rope_inv_freq(base, k.shape[-1])     # [..., 32], fp64 angles
    c, s = np.cos(phi), np.sin(phi)
    even, odd = k[..., 0::2], k[..., 1::2]
    out = np.empty_like(k)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


# ----------------------------------------------------------------------------
# append ([A] compression, [B] RoPE key, R6, R7)
# ----------------------------------------------------------------------------
def append_rows_exact(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray,
                      pos: np.ndarray, base: float) -> np.ndarray:
    """Latent rows before storage rounding, fp64 [n_tok, 576]:
    row = (W_DKV h) || RoPE(W_KR h, pos)."""
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, dtype=np.float64).T          # [n_tok, 512]
    k = h @ np.asarray(w_kr, dtype=np.float64).T           # [n_tok, 64]
    return np.concatenate([c, rope_rotate(k, pos, base)], axis=1)


def quantize_rows(rows: np.ndarray, dtype: str) -> Tuple[np.ndarray, Optional[np.ndarray], np.ndarray]:
    """Store exact rows in the cache dtype.

    Returns (stored, scale, dequantised): `stored` is the fp64 value of each
    element for f32/bf16 and the uint8 code for fp8; `scale` is the fp32 scale
    per row (fp8 only); `dequantised` is what a reader of the cache sees."""
    rows = np.asarray(rows, dtype=np.float64)
    if dtype == "f32":
        v = round_f32(rows)
        return v, None, v
    if dtype == "bf16":
        v = round_bf16(rows)
        return v, None, v
    if dtype == "fp8":
        amax = np.max(np.abs(rows), axis=1)
        scale = np.where(amax > 0, round_f32(amax / E4M3_MAX), 1.0)
        codes = e4m3_encode(rows / scale[:, None])
        deq = e4m3_decode(codes) * scale[:, None]
        return codes, scale, deq
    raise ValueError(dtype)


def widen_rows(rows, dtype: str, row_scale=None) -> np.ndarray:
    """fp64 view of stored cache rows: f32/bf16 values widened, fp8 codes
    decoded and multiplied by their row's scale."""
    if dtype == "fp8":
        codes = np.asarray(rows, dtype=np.uint8)
        sc = np.asarray(row_scale, dtype=np.float64)
        return e4m3_decode(codes) * sc[..., None]
    return np.asarray(rows, dtype=np.float64)


# ----------------------------------------------------------------------------
# decode: unabsorbed textbook attention ([A], [B], R1, R2, R4, R5)
# ----------------------------------------------------------------------------
def _scores(C: np.ndarray, R: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
            w_uk: np.ndarray) -> np.ndarray:
    K = C @ w_uk.T                          # K[t, i] = sum_j W_UK[i, j] C[t, j]
    return softmax_scale() * (K @ q_nope + R @ q_pe)


def attention_weights(C, R, q_nope, q_pe, w_uk) -> np.ndarray:
    """Softmax weights p[t] of one head over the sequence's tokens."""
    C = np.asarray(C, np.float64)
    s = _scores(C, np.asarray(R, np.float64), np.asarray(q_nope, np.float64),
                np.asarray(q_pe, np.float64), np.asarray(w_uk, np.float64))
    e = np.exp(s - s.max())
    return e / e.sum()


def decode_head(C: np.ndarray, R: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                w_uk: np.ndarray, w_uv: np.ndarray) -> Tuple[np.ndarray, float]:
    """o and lse for one (sequence, head).

    C [L, 512] latents, R [L, 64] shared RoPE keys, q_nope [128], q_pe [64],
    w_uk [128, 512], w_uv [512, 128]. K and V are expanded explicitly:
    K = C W_UK^T, V = C W_UV; s = sigma (K q_nope + R q_pe); p = softmax(s);
    o = p V; lse = max s + ln sum exp(s - max s)."""
    C = np.asarray(C, np.float64)
    R = np.asarray(R, np.float64)
    if C.shape[0] < 1:
        raise ValueError("decode over an empty sequence is undefined")
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    s = _scores(C, R, np.asarray(q_nope, np.float64), np.asarray(q_pe, np.float64), w_uk)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    V = C @ w_uv                            # V[t, i] = sum_j C[t, j] W_UV[j, i]
    o = (e / z) @ V
    return o, float(m + np.log(z))


def decode_sampled(rows64_of_seq, q_nope, q_pe, w_uk, w_uv,
                   pairs: Iterable[Tuple[int, int]]):
    """o [n, 128] and lse [n] for the listed (b, h) pairs.

    `rows64_of_seq(b)` returns the fp64 [L_b, 576] rows of sequence b."""
    pairs = list(pairs)
    out = np.zeros((len(pairs), D_V))
    lse = np.zeros(len(pairs))
    cur_b, rows = None, None
    for n, (b, h) in enumerate(pairs):
        if b != cur_b:
            rows, cur_b = rows64_of_seq(b), b
        out[n], lse[n] = decode_head(rows[:, :D_C], rows[:, D_C:], q_nope[b, h], q_pe[b, h],
                                     w_uk[h], w_uv[h])
    return out, lse


def decode_problem(rows64_of_seq, q_nope, q_pe, w_uk, w_uv, B: int, H: int):
    """Full o [B, H, 128] and lse [B, H]."""
    pairs = [(b, h) for b in range(B) for h in range(H)]
    o, lse = decode_sampled(rows64_of_seq, q_nope, q_pe, w_uk, w_uv, pairs)
    return o.reshape(B, H, D_V), lse.reshape(B, H)
