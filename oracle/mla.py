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
  R8  YaRN on the decoupled key [B gives scale 40, alpha 1, beta 32 and a
      160K target, but no formula]: the frequencies follow the published
      YaRN method ("NTK-by-parts" interpolation): for pair i with
      theta_i = base^(-2i/64) and wavelength 2*pi/theta_i, r_i = L / wavelength
      is the number of rotations over the original context L; the ramp
      gamma = clip((r_i - alpha) / (beta - alpha), 0, 1) mixes the
      interpolated and the original frequency,
      theta'_i = (1 - gamma) * theta_i / s + gamma * theta_i;
      L = target / s = 160K / 40 = 4096. The method's attention temperature
      multiplies the softmax scale by (0.1 ln s + 1)^2 (s > 1; 1 otherwise).
  R9  paged cache [the deployment guides name vLLM's PagedAttention and
      continuous batching as the serving engine's features (mlqm.cn guide,
      sections 3.2 "software environment" and 8.2 "deployment optimisation"),
      without a layout]: the cache is a pool of pages of P rows (P a multiple
      of the 32-token tile); sequence b's token t lives in row
      block_table[b][t // P] * P + t % P; rows are stored as in the contiguous
      cache, so attention over a paged cache equals attention over the
      sequence's rows gathered in token order.
  R11 the ~6-bit cache [reading card, "Method adaptation": elements quantised
      to about 6 bits on average; no format named]: OCP microscaling FP6 --
      e2m3 elements (sign, 2-bit exponent with bias 1, 3-bit mantissa, largest
      7.5) in blocks of 32 consecutive elements of a row, each block with one
      e8m0 scale 2^X, X = floor(log2(max|block|)) - 2 (so the block's largest
      element lies in [4, 8) before rounding), elements rounded to nearest
      even with saturation at 7.5; 18 blocks per 576-wide row. A stored row is
      464 bytes: the codes packed little-endian (element i takes bits
      6i .. 6i+5 of bytes 0..431), the 18 scale codes (bytes 432..449), zero
      padding to a multiple of 16 bytes (6.44 bits per element).
  R10 prefill / multi-query attention [the pages measure prompt processing
      beside generation -- over 100K prompt tokens/s on one 8-GPU node
      (DeepSeek-V2 reading card, "Evidence"; discosf explainer, throughput
      paragraph) -- but give no prefill formula]: the queries of sequence b
      are its last n_b positions, whose rows are already in the cache; the
      query at 0-based position p attends rows 0..p of its sequence (causal)
      with the decode score, softmax and output (R1, R2, R5); n_b = L_b is a
      whole-prompt prefill, n_b < L_b a chunk after a cached prefix.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .numerics import (round_bf16, round_f32, e4m3_decode, e4m3_encode, E4M3_MAX,
                       e2m3_decode, e2m3_encode, mx_block_exponent, pack6, unpack6, MX_BLOCK)

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


def yarn_inv_freq(base: float, scale: float, alpha: float, beta: float, orig_context: int,
                  d_r: int = D_R) -> np.ndarray:
    """YaRN frequencies theta'_i of the RoPE pairs, fp64 (R8): the number of
    rotations r_i of pair i over the original context decides between the
    original frequency (r_i >= beta: many rotations, kept), the frequency
    divided by the scale (r_i <= alpha: less than about one rotation,
    interpolated) and a linear mix of the two in between."""
    theta = rope_inv_freq(base, d_r)
    wavelength = 2.0 * np.pi / theta
    r = float(orig_context) / wavelength
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / scale + gamma * theta


def yarn_softmax_factor(scale: float) -> float:
    """Factor on the softmax scale from YaRN's attention temperature:
    sqrt(1/t) = 0.1 ln s + 1 scales both query and key, so the logits gain
    (0.1 ln s + 1)^2 (R8); 1 for s <= 1."""
    if scale <= 1.0:
        return 1.0
    m = 0.1 * np.log(np.float64(scale)) + 1.0
    return float(m * m)


def rope_rotate(k: np.ndarray, pos, base: float, inv_freq: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotate each interleaved pair (k[2i], k[2i+1]) of the last axis by
    pos * theta_i. `k` is [..., 64], `pos` broadcasts against k[..., 0];
    `inv_freq` replaces the plain frequencies (YaRN, R8)."""
    k = np.asarray(k, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    theta = rope_inv_freq(base, k.shape[-1]) if inv_freq is None else np.asarray(inv_freq, np.float64)
    phi = pos * theta                                # [..., 32], fp64 angles
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
                      pos: np.ndarray, base: float, inv_freq: Optional[np.ndarray] = None) -> np.ndarray:
    """Latent rows before storage rounding, fp64 [n_tok, 576]:
    row = (W_DKV h) || RoPE(W_KR h, pos) (with `inv_freq`: YaRN, R8)."""
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, dtype=np.float64).T          # [n_tok, 512]
    k = h @ np.asarray(w_kr, dtype=np.float64).T           # [n_tok, 64]
    return np.concatenate([c, rope_rotate(k, pos, base, inv_freq)], axis=1)


def paged_rows(rows: np.ndarray, block_table: np.ndarray, page_tokens: int, b: int,
               length: int) -> np.ndarray:
    """Sequence b's first `length` rows of a paged cache, in token order (R9):
    token t is row block_table[b][t // P] * P + t % P of `rows`."""
    t = np.arange(length)
    idx = np.asarray(block_table)[b, t // page_tokens].astype(np.int64) * page_tokens + t % page_tokens
    return np.asarray(rows)[idx]


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
    if dtype == "fp6":
        # R11: blocks of 32 along the row, one shared power-of-two exponent each
        n = rows.shape[0]
        blk = rows.reshape(n, -1, MX_BLOCK)
        x = mx_block_exponent(np.max(np.abs(blk), axis=2))          # [n, 18]
        codes = e2m3_encode(blk / np.ldexp(1.0, x)[..., None])         # exact scaling
        deq = (e2m3_decode(codes) * np.ldexp(1.0, x)[..., None]).reshape(n, -1)
        stored = np.zeros((n, FP6_ROW_BYTES), dtype=np.uint8)
        stored[:, :FP6_CODE_BYTES] = pack6(codes.reshape(n, -1))
        stored[:, FP6_CODE_BYTES:FP6_CODE_BYTES + D_ROW // MX_BLOCK] = x + 127
        return stored, None, deq
    raise ValueError(dtype)


FP6_CODE_BYTES = 432          # 576 six-bit codes
FP6_ROW_BYTES = 464           # codes, 18 scale codes, padding


def fp6_rows(stored: np.ndarray) -> np.ndarray:
    """fp64 values of stored fp6 cache rows [n, 464] (R11): e2m3 codes
    unpacked from bytes 0..431, each times 2^(code - 127) of its block's
    scale byte (bytes 432..449)."""
    stored = np.asarray(stored, dtype=np.uint8)
    codes = unpack6(stored[:, :FP6_CODE_BYTES])
    n = codes.shape[0]
    blk = e2m3_decode(codes).reshape(n, -1, MX_BLOCK)
    x = stored[:, FP6_CODE_BYTES:FP6_CODE_BYTES + D_ROW // MX_BLOCK].astype(np.int64) - 127
    return (blk * np.ldexp(1.0, x)[..., None]).reshape(n, -1)


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


# ----------------------------------------------------------------------------
# prefill: causal multi-query attention (R10 with R1, R2, R5)
# ----------------------------------------------------------------------------
def prefill_head(C: np.ndarray, R: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                 w_uk: np.ndarray, w_uv: np.ndarray, pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """o [n, 128] and lse [n] for n queries of one (sequence, head).

    C [L, 512] and R [L, 64] are the sequence's rows, q_nope [n, 128] and
    q_pe [n, 64] the queries, pos [n] their 0-based positions (< L). As in
    decode, K = C W_UK^T and V = C W_UV are expanded explicitly; query i's
    scores over rows t > pos[i] are excluded (weight 0)."""
    C = np.asarray(C, np.float64)
    R = np.asarray(R, np.float64)
    pos = np.asarray(pos, np.int64)
    L = C.shape[0]
    if len(pos) and (pos.min() < 0 or pos.max() >= L):
        raise ValueError("query position outside the sequence")
    K = C @ np.asarray(w_uk, np.float64).T          # K[t, i] = sum_j W_UK[i, j] C[t, j]
    V = C @ np.asarray(w_uv, np.float64)            # V[t, i] = sum_j C[t, j] W_UV[j, i]
    s = softmax_scale() * (np.asarray(q_nope, np.float64) @ K.T + np.asarray(q_pe, np.float64) @ R.T)
    s[np.arange(L)[None, :] > pos[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ V, (m + np.log(z))[:, 0]


def prefill_positions(seq_len: int, n_q: int) -> np.ndarray:
    """Positions of a sequence's n_q queries: its last n_q slots (R10)."""
    if not 0 <= n_q <= seq_len:
        raise ValueError("a sequence has at most seq_len queries")
    return np.arange(seq_len - n_q, seq_len, dtype=np.int64)


def prefill_problem(rows64_of_seq, seq_len, q_start, q_nope, q_pe, w_uk, w_uv,
                    heads: Optional[Sequence[int]] = None):
    """o [n_q, H, 128] and lse [n_q, H] (heads not listed stay 0 / -inf).

    Query rows q_start[b] .. q_start[b+1]-1 belong to sequence b."""
    n_q, H = q_nope.shape[0], q_nope.shape[1]
    heads = range(H) if heads is None else heads
    out = np.zeros((n_q, H, D_V))
    lse = np.full((n_q, H), -np.inf)
    for b in range(len(seq_len)):
        q0, q1 = int(q_start[b]), int(q_start[b + 1])
        if q1 == q0:
            continue
        rows = rows64_of_seq(b)
        pos = prefill_positions(int(seq_len[b]), q1 - q0)
        for h in heads:
            out[q0:q1, h], lse[q0:q1, h] = prefill_head(rows[:, :D_C], rows[:, D_C:],
                                                        q_nope[q0:q1, h], q_pe[q0:q1, h],
                                                        w_uk[h], w_uv[h], pos)
    return out, lse
