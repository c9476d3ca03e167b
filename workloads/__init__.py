"""Seeded synthetic inputs for MLA decode/append, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module only *draws* inputs and lays them out; it holds none of the
method's arithmetic (no projection, no RoPE, no attention, no quantisation
rule). Values that a GPU kernel will read in bf16 or fp8 are cast with
torch's own CPU casts (library routines), so the oracle and the HIP path see
exactly the same numbers and neither side's codec is involved in making them.

Workloads follow the shapes of DeepSeek-V2 (128 heads) and DeepSeek-V2-Lite
(16 heads) decode: a latent row per cached token holds c_KV (d_c = 512) and a
decoupled RoPE key (d_R = 64), 576 elements in all (DeepSeek-V2 reading card,
"Method adaptation"; discosf explainer, "long-context bottleneck" and
"decoupled RoPE" sections). The pages measure on production request-length
distributions that are not available; uniform length draws stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

D_C = 512      # latent width d_c
D_R = 64       # decoupled RoPE key width d_R
D_ROW = D_C + D_R
D_NOPE = 128   # per-head non-RoPE query/key width
D_V = 128      # per-head value width


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int             # position in the workload list; also the RNG seed
    B: int                 # sequences
    H: int                 # heads
    lo: int                # per-sequence cached length drawn uniformly in [lo, hi]
    hi: int
    cache: str             # "f32" | "bf16" | "fp8"
    act: str               # dtype of q, weights and out: "f32" | "bf16"
    append: bool = False   # one appended token per sequence before decode
    d_model: int = 2048
    rope_base: float = 10000.0

    @property
    def seed(self) -> int:
        return self.index


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 0, B=1, H=16, lo=256, hi=256, cache="f32", act="f32"),
        Workload("v2lite_bf16", 1, B=64, H=16, lo=1024, hi=4096, cache="bf16", act="bf16",
                 append=True, d_model=2048, rope_base=10000.0),
        Workload("v2_bf16", 2, B=32, H=128, lo=2048, hi=8192, cache="bf16", act="bf16"),
        Workload("long_bf16", 3, B=4, H=128, lo=131072, hi=131072, cache="bf16", act="bf16"),
        Workload("fp8_cache", 4, B=128, H=128, lo=512, hi=4096, cache="fp8", act="bf16"),
        # the ~6-bit cache: e2m3 codes in blocks of 32 with one e8m0 scale each
        Workload("fp6_cache", 5, B=128, H=128, lo=512, hi=4096, cache="fp6", act="bf16"),
    ]
}
# bytes of a stored row (and of its scale record) per cache format
ROW_BYTES = {"f32": 2304, "bf16": 1152, "fp8": 576, "fp6": 464}
FP6_CODE_BYTES, FP6_SCALES_PER_ROW = 432, 18     # an fp6 row: codes, block scales, padding

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}

# rows left unused after each sequence's capacity; they hold a canary pattern
CANARY_ROWS = 3
# fp8 synthetic cache: codes come from torch's e4m3fn cast of FP8_SPREAD * z
# (clamped to the finite range) and each token gets its own positive scale
FP8_SPREAD = 100.0


@dataclasses.dataclass
class Problem:
    """One synthetic MLA decode problem, all tensors on the host (CPU).

    Cache tensors are in the storage dtype the GPU uses; the fp64 view the
    oracle needs is obtained by widening them (fp8: decoding + scaling)."""
    wl: Workload
    seq_len: np.ndarray          # [B] int32, cached length each sequence is decoded over
    seq_start: np.ndarray        # [B] int64, first row of each sequence
    seq_capacity: np.ndarray     # [B] int32, rows reserved per sequence
    total_rows: int
    rows: torch.Tensor           # [total_rows, 576] f32 | bf16 | uint8 (fp8 codes)
    row_scale: Optional[torch.Tensor]   # [total_rows] f32 (fp8 only)
    q_nope: torch.Tensor         # [B, H, 128]  act dtype
    q_pe: torch.Tensor           # [B, H, 64]   act dtype
    w_uk: torch.Tensor           # [H, 128, 512] act dtype
    w_uv: torch.Tensor           # [H, 512, 128] act dtype
    # append inputs (one token per sequence at position seq_len-1), or None
    h: Optional[torch.Tensor] = None       # [n_tok, d_model]
    w_dkv: Optional[torch.Tensor] = None   # [512, d_model]
    w_kr: Optional[torch.Tensor] = None    # [64, d_model]
    tok_seq: Optional[np.ndarray] = None   # [n_tok] int32
    tok_pos: Optional[np.ndarray] = None   # [n_tok] int32

    @property
    def T(self) -> int:
        return int(self.seq_len.astype(np.int64).sum())


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _to(x: np.ndarray, dt: str) -> torch.Tensor:
    return torch.from_numpy(x).to(TORCH_DTYPE[dt])


def fp8_codes_from_normal(z: np.ndarray) -> torch.Tensor:
    """uint8 e4m3fn codes of clamp(FP8_SPREAD*z) made by torch's CPU cast."""
    t = torch.from_numpy(z)
    t = (t * FP8_SPREAD).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8)


def make_problem(wl: Workload, seed: Optional[int] = None, *, B: Optional[int] = None,
                 lengths: Optional[np.ndarray] = None, H: Optional[int] = None,
                 canary: int = CANARY_ROWS) -> Problem:
    """Draw a problem for workload `wl`.

    Draw order (fixed): lengths, cache rows (c_KV and k_pe together as one
    [rows, 576] normal draw; fp8 adds one uniform per row for the scale),
    q_nope, q_pe, W_UK, W_UV, then for append h, W_DKV, W_KR.
    `B`, `lengths` and `H` override the workload's values for small cases."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    if lengths is None:
        seq_len = rng.integers(wl.lo, wl.hi, size=B, endpoint=True).astype(np.int32)
    else:
        seq_len = np.asarray(lengths, dtype=np.int32).copy()
        assert seq_len.shape == (B,)
    cap = (seq_len.astype(np.int64) + canary)
    seq_start = np.zeros(B, dtype=np.int64)
    if B > 1:
        seq_start[1:] = np.cumsum(cap)[:-1]
    total_rows = int(cap.sum())

    row_scale = None
    if wl.cache == "fp6":
        rows = fp6_rows_random(rng, total_rows)
    else:
        z = _normal(rng, (total_rows, D_ROW))
        if wl.cache == "fp8":
            rows = fp8_codes_from_normal(z)
            u = rng.uniform(-0.5, 0.5, size=total_rows)
            row_scale = torch.from_numpy((np.exp(u) / FP8_SPREAD).astype(np.float32))
        else:
            rows = _to(z, wl.cache)
        del z

    act = wl.act
    w_std = 1.0 / np.sqrt(D_C)   # fan_in of both up-projections is d_c = 512
    q_nope = _to(_normal(rng, (B, H, D_NOPE)), act)
    q_pe = _to(_normal(rng, (B, H, D_R)), act)
    w_uk = _to(_normal(rng, (H, D_NOPE, D_C), w_std), act)
    w_uv = _to(_normal(rng, (H, D_C, D_V), w_std), act)

    p = Problem(wl=wl, seq_len=seq_len, seq_start=seq_start,
                seq_capacity=cap.astype(np.int32), total_rows=total_rows, rows=rows,
                row_scale=row_scale, q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv)
    if wl.append:
        dm = wl.d_model
        a_std = 1.0 / np.sqrt(dm)
        p.h = _to(_normal(rng, (B, dm)), act)
        p.w_dkv = _to(_normal(rng, (D_C, dm), a_std), act)
        p.w_kr = _to(_normal(rng, (D_R, dm), a_std), act)
        p.tok_seq = np.arange(B, dtype=np.int32)
        p.tok_pos = (seq_len - 1).astype(np.int32)
    return p


def canary_mask(p: Problem) -> np.ndarray:
    """Boolean [total_rows]: True for rows no sequence's length covers."""
    m = np.ones(p.total_rows, dtype=bool)
    for b in range(len(p.seq_len)):
        s = int(p.seq_start[b])
        m[s:s + int(p.seq_len[b])] = False
    return m


def algorithmic_bytes(p: Problem) -> dict:
    """Bytes the decode must move (cache rows + scales, both weights, q, out)."""
    e_a = {"f32": 4, "bf16": 2}[p.wl.act]
    B, H = p.q_nope.shape[0], p.q_nope.shape[1]
    scale_bytes = {"fp8": 4}.get(p.wl.cache, 0)            # (fp6 rows hold their scales)
    cache = p.T * (ROW_BYTES[p.wl.cache] + scale_bytes)
    weights = 2 * H * D_NOPE * D_C * e_a
    q = B * H * (D_NOPE + D_R) * e_a
    out = B * H * D_V * e_a
    return {"cache": cache, "weights": weights, "q": q, "out": out,
            "total": cache + weights + q + out}


def algorithmic_flops(p: Problem) -> dict:
    B, H = p.q_nope.shape[0], p.q_nope.shape[1]
    attn = 2 * H * (D_ROW + D_C) * p.T
    absorb = 4 * B * H * D_NOPE * D_C
    return {"attention": attn, "absorb_project": absorb, "total": attn + absorb}


def fp6_rows_random(rng, n: int) -> torch.Tensor:
    """n stored fp6 rows of random content: any byte string is a valid packed
    run of 6-bit codes; block scale codes 120..127 (2^-7 .. 1); zero padding."""
    r = np.zeros((n, ROW_BYTES["fp6"]), dtype=np.uint8)
    r[:, :FP6_CODE_BYTES] = rng.integers(0, 256, size=(n, FP6_CODE_BYTES), dtype=np.uint8)
    r[:, FP6_CODE_BYTES:FP6_CODE_BYTES + FP6_SCALES_PER_ROW] = rng.integers(
        120, 128, size=(n, FP6_SCALES_PER_ROW), dtype=np.uint8)
    return torch.from_numpy(r)


# ----------------------------------------------------------------------------
# prefill / multi-query problems: the last n_b positions of each sequence are
# queries (n_b = L_b: a whole prompt; n_b < L_b: a chunk after a cached prefix)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    index: int             # RNG seed
    B: int
    H: int
    lo: int                # sequence length drawn uniformly in [lo, hi]
    hi: int
    cache: str             # "bf16" | "fp8" | "fp6"
    chunk: int = 0         # 0: every position is a query; else n_b = min(chunk, L_b)


PREFILL_WORKLOADS = {
    w.name: w for w in [
        # DeepSeek-V2 attention shape (128 heads), four prompts of 2K-4K tokens
        PrefillWorkload("prefill_bf16", 10, B=4, H=128, lo=2048, hi=4096, cache="bf16"),
        # a 512-token chunk after a cached prefix, fp8 cache
        PrefillWorkload("prefill_chunk_fp8", 11, B=8, H=128, lo=1024, hi=6144, cache="fp8",
                        chunk=512),
        # the same chunked shape over the ~6-bit (microscaling FP6) cache
        PrefillWorkload("prefill_chunk_fp6", 12, B=8, H=128, lo=1024, hi=6144, cache="fp6",
                        chunk=512),
    ]
}


@dataclasses.dataclass
class PrefillProblem:
    """One synthetic prefill problem (host tensors)."""
    wl: PrefillWorkload
    seq_len: np.ndarray          # [B] int32
    seq_start: np.ndarray        # [B] int64
    seq_capacity: np.ndarray     # [B] int32
    total_rows: int
    rows: torch.Tensor           # [total_rows, 576] bf16 | uint8 codes
    row_scale: Optional[torch.Tensor]
    q_start: np.ndarray          # [B + 1] int32: queries of b are rows q_start[b]..q_start[b+1]-1
    q_nope: torch.Tensor         # [n_q, H, 128] bf16
    q_pe: torch.Tensor           # [n_q, H, 64] bf16
    w_uk: torch.Tensor           # [H, 128, 512] bf16
    w_uv: torch.Tensor           # [H, 512, 128] bf16

    @property
    def n_q(self) -> int:
        return int(self.q_start[-1])

    @property
    def T(self) -> int:
        return int(self.seq_len.astype(np.int64).sum())


def make_prefill_problem(wl: PrefillWorkload, seed: Optional[int] = None, *,
                         lengths: Optional[Sequence[int]] = None,
                         n_queries: Optional[Sequence[int]] = None,
                         H: Optional[int] = None, canary: int = CANARY_ROWS) -> PrefillProblem:
    """Draw a prefill problem. Draw order (fixed): lengths, cache rows (fp8:
    then one uniform per row for the scale; fp6: code bytes, then scale codes),
    q_nope, q_pe, W_UK, W_UV."""
    rng = np.random.Generator(np.random.PCG64(wl.index if seed is None else seed))
    H = wl.H if H is None else H
    if lengths is None:
        seq_len = rng.integers(wl.lo, wl.hi, size=wl.B, endpoint=True).astype(np.int32)
    else:
        seq_len = np.asarray(lengths, dtype=np.int32).copy()
    B = len(seq_len)
    if n_queries is None:
        nq = seq_len.copy() if wl.chunk == 0 else np.minimum(seq_len, wl.chunk).astype(np.int32)
    else:
        nq = np.asarray(n_queries, dtype=np.int32).copy()
        assert nq.shape == (B,) and np.all((nq >= 0) & (nq <= seq_len))
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(nq)
    cap = seq_len.astype(np.int64) + canary
    seq_start = np.zeros(B, dtype=np.int64)
    if B > 1:
        seq_start[1:] = np.cumsum(cap)[:-1]
    total_rows = int(cap.sum())
    row_scale = None
    if wl.cache == "fp6":
        rows = fp6_rows_random(rng, total_rows)
    else:
        z = _normal(rng, (total_rows, D_ROW))
        if wl.cache == "fp8":
            rows = fp8_codes_from_normal(z)
            u = rng.uniform(-0.5, 0.5, size=total_rows)
            row_scale = torch.from_numpy((np.exp(u) / FP8_SPREAD).astype(np.float32))
        else:
            rows = _to(z, wl.cache)
        del z
    n_q = int(q_start[-1])
    w_std = 1.0 / np.sqrt(D_C)
    q_nope = _to(_normal(rng, (n_q, H, D_NOPE)), "bf16")
    q_pe = _to(_normal(rng, (n_q, H, D_R)), "bf16")
    w_uk = _to(_normal(rng, (H, D_NOPE, D_C), w_std), "bf16")
    w_uv = _to(_normal(rng, (H, D_C, D_V), w_std), "bf16")
    return PrefillProblem(wl=wl, seq_len=seq_len, seq_start=seq_start,
                          seq_capacity=cap.astype(np.int32), total_rows=total_rows, rows=rows,
                          row_scale=row_scale, q_start=q_start, q_nope=q_nope, q_pe=q_pe,
                          w_uk=w_uk, w_uv=w_uv)


def prefill_flops(p: PrefillProblem) -> dict:
    """Matrix work of a prefill step: the up-projection of every cached row
    to per-head K (128) and V (128) from its 512-wide latent, and the causal
    attention (score over 128 + 64 dims, values over 128) counted over the
    (query, row) pairs a query may see."""
    H = p.q_nope.shape[1]
    kv = 2.0 * p.T * D_C * (D_NOPE + D_V) * H
    pairs = 0
    for b in range(len(p.seq_len)):
        L = int(p.seq_len[b])
        n = int(p.q_start[b + 1] - p.q_start[b])
        pos = np.arange(L - n, L, dtype=np.int64)
        pairs += int((pos + 1).sum())
    attn = 2.0 * pairs * H * (D_NOPE + D_R + D_V)
    return {"kv": kv, "attn": attn, "total": kv + attn, "pairs": pairs}
