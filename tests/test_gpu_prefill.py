"""GPU parity of mla_prefill (causal multi-query attention) against the fp64
oracle, through the C ABI.

Small cases compare every output: whole-prompt prefill over ragged lengths
(1 row, partial and several 64-row blocks), chunks after a cached prefix,
several 256-query blocks per sequence, sequences without queries between
others, fp8 and fp6 caches, odd head counts, paged caches (bit for bit equal
to the contiguous ones). The full-size case (the benchmark's
shape: 128 heads, four prompts of 2K-4K tokens) compares every query of
sampled (sequence, head) pairs. Bounds: rel-L2 2e-2 on o (bf16 cache), 4e-2
(fp8 and fp6 caches, against the oracle on the dequantised rows); |lse error|
<= 1e-2 + 1e-3 |lse|."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.problem import PrefillOracleView
from tests.gpu_util import TOL, log, rel_l2

pytestmark = pytest.mark.gpu


class DevicePrefill:
    def __init__(self, p, device="cuda"):
        import head_latent_attention_14_amd as mla
        self.mla = mla
        self.p = p
        dev = torch.device(device)
        scale = p.row_scale.to(dev) if p.row_scale is not None else None
        self.cache = mla.LatentCache(rows=p.rows.to(dev), seq_start=torch.from_numpy(p.seq_start).to(dev),
                                     seq_capacity=torch.from_numpy(p.seq_capacity).to(dev),
                                     row_scale=scale)
        self.seq_len = torch.from_numpy(p.seq_len).to(dev)
        self.q_start = torch.from_numpy(p.q_start).to(dev)
        self.q_nope = p.q_nope.to(dev)
        self.q_pe = p.q_pe.to(dev)
        self.w_uk = p.w_uk.to(dev)
        self.w_uv = p.w_uv.to(dev)
        n_q, H = p.q_nope.shape[:2]
        self.H = H
        self.max_kv_rows = max(p.T, 1)
        self.out = torch.empty(n_q, H, 128, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(n_q, H, dtype=torch.float32, device=dev)
        self.ws = mla.alloc_prefill_workspace(self.cache, H, n_q, self.max_kv_rows)

    def run(self, poison=True):
        if poison:
            self.out.fill_(float("nan"))
            self.lse.fill_(float("nan"))
            self.ws.fill_(0xFF)
        self.mla.mla_prefill(self.cache, self.seq_len, self.q_start, self.max_kv_rows, self.q_nope,
                             self.q_pe, self.w_uk, self.w_uv, 1.0 / math.sqrt(192.0), self.out,
                             self.lse, self.ws)
        torch.cuda.synchronize()
        return self.out.double().cpu().numpy(), self.lse.double().cpu().numpy()


def _check(p, o, lse, heads=None, label=""):
    view = PrefillOracleView(p)
    ro, rl = view.prefill(heads)
    hs = list(range(p.q_nope.shape[1])) if heads is None else list(heads)
    tol = TOL[p.wl.cache]
    got, ref = o[:, hs], ro[:, hs]
    err = rel_l2(got, ref)
    lerr = np.abs(lse[:, hs] - rl[:, hs])
    bound = 1e-2 + 1e-3 * np.abs(rl[:, hs])
    log(f"  {label} rel-L2 {err:.3e} (bound {tol}), max abs {np.abs(got - ref).max():.3e}, "
        f"lse max err {lerr.max():.3e}")
    assert np.all(np.isfinite(got))
    assert err <= tol
    assert np.all(lerr <= bound)
    # every sequence on its own meets the bound too
    for b in range(len(p.seq_len)):
        q0, q1 = int(p.q_start[b]), int(p.q_start[b + 1])
        if q1 > q0:
            assert rel_l2(got[q0:q1], ref[q0:q1]) <= tol, b
    return err


@pytest.mark.parametrize("cache", ["bf16", "fp8", "fp6"])
def test_prefill_whole_prompts_small(cache):
    name = {"bf16": "prefill_bf16", "fp8": "prefill_chunk_fp8", "fp6": "prefill_chunk_fp6"}[cache]
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS[name], lengths=[1, 37, 300, 64],
                               n_queries=[1, 37, 300, 64], H=16)
    log(f"[prefill small] {cache} lengths={p.seq_len.tolist()} H=16")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label=cache)


def test_prefill_chunks_after_a_prefix():
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_bf16"], lengths=[700, 1300, 90, 513],
                               n_queries=[100, 300, 90, 1], H=8, seed=3)
    log(f"[prefill chunks] lengths={p.seq_len.tolist()} queries={np.diff(p.q_start).tolist()}")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label="chunks")


def test_prefill_several_query_blocks_per_sequence():
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_bf16"], lengths=[600, 257],
                               n_queries=[600, 257], H=8, seed=4)
    log(f"[prefill blocks] lengths={p.seq_len.tolist()}")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label="blocks")


def test_prefill_sequences_without_queries_between_others():
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_bf16"], lengths=[50, 80, 3, 200, 10],
                               n_queries=[0, 80, 0, 20, 0], H=4, seed=5)
    log(f"[prefill gaps] queries={np.diff(p.q_start).tolist()}")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label="gaps")


@pytest.mark.parametrize("H", [1, 3, 128])
def test_prefill_head_counts(H):
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_bf16"], lengths=[130, 66],
                               n_queries=[130, 40], H=H, seed=6)
    log(f"[prefill heads] H={H}")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label=f"H={H}")


def test_prefill_fp8_chunk_small():
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_chunk_fp8"], lengths=[900, 300],
                               n_queries=[300, 300], H=16, seed=7)
    log("[prefill fp8 chunk]")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label="fp8 chunk")


def test_prefill_fp6_chunk_small():
    # rows widened from microscaling FP6 (block scales applied) before the
    # up-projection; the RoPE key from the last two blocks of each row
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_chunk_fp6"], lengths=[900, 300, 129],
                               n_queries=[300, 300, 1], H=16, seed=9)
    log("[prefill fp6 chunk]")
    o, lse = DevicePrefill(p).run()
    _check(p, o, lse, label="fp6 chunk")


@pytest.mark.parametrize("name,P", [("prefill_bf16", 32), ("prefill_chunk_fp8", 64),
                                    ("prefill_chunk_fp6", 32)])
def test_prefill_paged_equals_contiguous(name, P):
    # the same rows in shuffled P-row pages of a larger pool (unused rows
    # random): mla_prefill_paged equals mla_prefill bit for bit
    from tests.test_gpu_paged import _page
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS[name], lengths=[700, 33, 300, 129],
                               n_queries=[300, 33, 1, 129], H=16, seed=10)
    d = DevicePrefill(p)
    o, lse = d.run()
    pc = _page(d, P, seed=P)
    out = torch.full_like(d.out, float("nan"))
    lse_p = torch.full_like(d.lse, float("nan"))
    ws = d.mla.alloc_prefill_workspace(pc, d.H, out.shape[0], d.max_kv_rows)
    ws.fill_(0xFF)
    d.mla.mla_prefill(pc, d.seq_len, d.q_start, d.max_kv_rows, d.q_nope, d.q_pe, d.w_uk, d.w_uv,
                      1.0 / math.sqrt(192.0), out, lse_p, ws)
    torch.cuda.synchronize()
    log(f"[prefill paged] {name} P={P}")
    assert np.array_equal(out.double().cpu().numpy(), o)
    assert np.array_equal(lse_p.double().cpu().numpy(), lse)
    _check(p, o, lse, label=f"{name} paged")


def test_prefill_repeatable():
    p = W.make_prefill_problem(W.PREFILL_WORKLOADS["prefill_bf16"], lengths=[400, 77],
                               n_queries=[400, 77], H=8, seed=8)
    d = DevicePrefill(p)
    o1, l1 = d.run()
    o2, l2 = d.run()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", list(W.PREFILL_WORKLOADS))
def test_prefill_full_size_sampled(name):
    """At the benchmark's shape: every query of 4 heads (of 128)."""
    wl = W.PREFILL_WORKLOADS[name]
    p = W.make_prefill_problem(wl)
    log(f"[prefill full] {name} lengths={p.seq_len.tolist()} n_q={p.n_q}")
    o, lse = DevicePrefill(p).run()
    assert np.all(np.isfinite(o))
    _check(p, o, lse, heads=[0, 37, 64, 127], label=name)
