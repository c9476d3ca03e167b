"""Run the oracle on a synthetic problem from `workloads` (test infrastructure only).

The oracle reads the same stored values the GPU reads (bf16/fp32 values
widened to fp64; fp8 codes decoded and scaled in fp64). When the problem has
an append step, the oracle computes the appended rows itself (exact fp64,
then rounded to the cache dtype by its own codec) and decodes over those.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Tuple

import numpy as np
import torch

from . import mla
from .numerics import e4m3_decode


def _np64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.uint8:
        raise TypeError("codes are not values")
    return t.to(torch.float64).numpy()


class OracleView:
    """fp64 view of a `workloads.Problem`, with the append applied by the oracle."""

    def __init__(self, p, apply_append: bool = True):
        self.p = p
        self.dtype = p.wl.cache
        self.q_nope = _np64(p.q_nope)
        self.q_pe = _np64(p.q_pe)
        self.w_uk = _np64(p.w_uk)
        self.w_uv = _np64(p.w_uv)
        self.appended: Dict[int, np.ndarray] = {}
        self.append_stored = None
        if apply_append and p.h is not None:
            exact = mla.append_rows_exact(_np64(p.h), _np64(p.w_dkv), _np64(p.w_kr),
                                          p.tok_pos.astype(np.float64), p.wl.rope_base)
            stored, scale, deq = mla.quantize_rows(exact, self.dtype)
            self.append_exact = exact
            self.append_stored = (stored, scale, deq)
            for n in range(len(p.tok_seq)):
                row = int(p.seq_start[p.tok_seq[n]]) + int(p.tok_pos[n])
                self.appended[row] = deq[n]

    def rows64(self, b: int) -> np.ndarray:
        p = self.p
        s, L = int(p.seq_start[b]), int(p.seq_len[b])
        sl = p.rows[s:s + L]
        if self.dtype == "fp8":
            codes = sl.numpy()
            sc = p.row_scale[s:s + L].to(torch.float64).numpy()
            out = e4m3_decode(codes) * sc[:, None]
        elif self.dtype == "fp6":
            out = mla.fp6_rows(sl.numpy())
        else:
            out = sl.to(torch.float64).numpy()
        for r, v in self.appended.items():
            if s <= r < s + L:
                out = out.copy() if not out.flags.writeable else out
                out[r - s] = v
        return out

    def decode(self, pairs: Optional[Iterable[Tuple[int, int]]] = None):
        """(o, lse): full [B,H,128]/[B,H] when `pairs` is None, else sampled."""
        B, H = self.q_nope.shape[0], self.q_nope.shape[1]
        if pairs is None:
            return mla.decode_problem(self.rows64, self.q_nope, self.q_pe, self.w_uk,
                                      self.w_uv, B, H)
        return mla.decode_sampled(self.rows64, self.q_nope, self.q_pe, self.w_uk,
                                  self.w_uv, pairs)


class PrefillOracleView:
    """fp64 view of a `workloads.PrefillProblem` (no append step)."""

    def __init__(self, p):
        self.p = p
        self.dtype = p.wl.cache
        self.q_nope = _np64(p.q_nope)
        self.q_pe = _np64(p.q_pe)
        self.w_uk = _np64(p.w_uk)
        self.w_uv = _np64(p.w_uv)

    def rows64(self, b: int) -> np.ndarray:
        p = self.p
        s, L = int(p.seq_start[b]), int(p.seq_len[b])
        sl = p.rows[s:s + L]
        if self.dtype == "fp8":
            return e4m3_decode(sl.numpy()) * p.row_scale[s:s + L].to(torch.float64).numpy()[:, None]
        if self.dtype == "fp6":
            return mla.fp6_rows(sl.numpy())
        return sl.to(torch.float64).numpy()

    def prefill(self, heads=None):
        """(o [n_q, H, 128], lse [n_q, H]); heads not in `heads` stay 0 / -inf."""
        return mla.prefill_problem(self.rows64, self.p.seq_len, self.p.q_start, self.q_nope,
                                   self.q_pe, self.w_uk, self.w_uv, heads)
