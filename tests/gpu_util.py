"""Helpers shared by the GPU tests: move a synthetic problem to the device,
run libmla on it, and compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import workloads as W

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 4e-2, "fp6": 4e-2}     # rel-L2 bounds on o[B,H,128]

# Unit roundoff of the absorbed query q_lat = W_UK[h]^T q_nope as the kernels
# hold it: fp32 for the f32 cache, bf16 (8 significant bits) otherwise.
Q_LAT_U = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "fp8": 2.0 ** -8, "fp6": 2.0 ** -8}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceProblem:
    def __init__(self, p: W.Problem, device="cuda"):
        import head_latent_attention_14_amd as mla
        self.mla = mla
        self.p = p
        dev = torch.device(device)
        self.dev = dev
        rows = p.rows.to(dev)
        scale = p.row_scale.to(dev) if p.row_scale is not None else None
        self.cache = mla.LatentCache(rows=rows, seq_start=torch.from_numpy(p.seq_start).to(dev),
                                     seq_capacity=torch.from_numpy(p.seq_capacity).to(dev),
                                     row_scale=scale)
        self.seq_len = torch.from_numpy(p.seq_len).to(dev)
        self.q_nope = p.q_nope.to(dev)
        self.q_pe = p.q_pe.to(dev)
        self.w_uk = p.w_uk.to(dev)
        self.w_uv = p.w_uv.to(dev)
        B, H = p.q_nope.shape[:2]
        self.B, self.H = B, H
        self.out = torch.empty(B, H, 128, dtype=p.q_nope.dtype, device=dev)
        self.lse = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.ws = mla.alloc_workspace(self.cache, H, p.q_nope.dtype)
        if p.h is not None:
            self.h = p.h.to(dev)
            self.w_dkv = p.w_dkv.to(dev)
            self.w_kr = p.w_kr.to(dev)
            self.tok_seq = torch.from_numpy(p.tok_seq).to(dev)
            self.tok_pos = torch.from_numpy(p.tok_pos).to(dev)

    def append(self):
        self.mla.mla_append(self.cache, self.h, self.w_dkv, self.w_kr, self.tok_seq, self.tok_pos,
                            self.p.wl.rope_base)

    def decode(self, poison=False):
        if poison:
            self.out.fill_(float("nan"))
            self.lse.fill_(float("nan"))
            self.ws.fill_(0xFF)        # NaN patterns in every fp32 slot
        self.mla.mla_decode(self.cache, self.seq_len, self.q_nope, self.q_pe, self.w_uk, self.w_uv,
                            1.0 / math.sqrt(192.0), self.out, self.lse, self.ws)

    def step(self, poison=False):
        if self.p.h is not None:
            self.append()
        self.decode(poison)
        torch.cuda.synchronize()
        return self.out.to(torch.float64).cpu().numpy(), self.lse.to(torch.float64).cpu().numpy()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def lse_bounds(view, pairs, cache: str) -> np.ndarray:
    """Per-(b, h) bound on |lse_gpu - lse_oracle|.

    The kernels' dominant lse error is the rounding of q_lat (unit roundoff u,
    Q_LAT_U) feeding every score: s_t moves by sigma * sum_i d_i q_i c_t,i with
    |d_i| <= u, the d_i independent roundings, so its standard deviation is at
    most sigma * u / sqrt(3) * sqrt(sum_i q_i^2 c_t,i^2). lse moves by a
    softmax-weighted mean of those shifts, so 6 of those deviations at the
    worst token bound it; 1e-4 (1 + |lse|) covers the fp32 accumulation, exp2
    and log of the kernels (f32: 1e-5)."""
    u = Q_LAT_U[cache]
    sigma = 1.0 / math.sqrt(192.0)
    out = np.empty(len(pairs))
    sq, cur = None, None
    for n, (b, h) in enumerate(pairs):
        if b != cur:
            sq, cur = view.rows64(b)[:, :512] ** 2, b
        q_lat = view.w_uk[h].T @ view.q_nope[b, h]
        dev = math.sqrt(float((sq @ (q_lat ** 2)).max())) if len(sq) else 0.0
        out[n] = 6.0 * sigma * u / math.sqrt(3.0) * dev
    return out


def check_lse(got, ref, view, pairs, cache: str, what: str = "") -> float:
    """Assert the lse bound on every listed pair; return the largest
    |error| / bound."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    bound = lse_bounds(view, pairs, cache) + (1e-5 if cache == "f32" else 1e-4) * (1 + np.abs(ref))
    err = np.abs(got - ref)
    worst = float((err / bound).max()) if len(err) else 0.0
    log(f"  lse max abs err {err.max() if len(err) else 0:.3e}, worst err/bound {worst:.3f} {what}")
    assert np.all(err <= bound), (what, int(np.argmax(err / bound)), float(err.max()))
    return worst
