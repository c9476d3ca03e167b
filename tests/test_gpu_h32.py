"""GPU parity of the one-wave-per-SIMD 128-head decode kernel (MLA_H32=1:
`mla_attn_h32_kernel`, bf16 cache, heads in multiples of 128) against the
fp64 oracle, at the bf16 bound (rel-L2 2e-2 on o).

Cases: every output of a small ragged problem (1 token, partial tiles,
several tiles with a ragged tail) at 128 and 256 heads; the V2 and 128K
shapes at full size (every head of sampled sequences: the 128K sequences are
split over many workers); empty sequences between others; bitwise repeats;
a paged cache equal to the contiguous one bit for bit; and agreement with the
default pair kernel to the rounding of the two summation orders."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.problem import OracleView
from tests.gpu_util import TOL, DeviceProblem, check_lse, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def h32(monkeypatch):
    monkeypatch.setenv("MLA_H32", "1")


def _problem(lengths, H=128, seed=None, name="v2_bf16"):
    lengths = np.array(lengths)
    return W.make_problem(W.WORKLOADS[name], seed=seed, B=len(lengths), lengths=lengths, H=H)


def _check_all(p, o, lse, label):
    view = OracleView(p)
    ro, rl = view.decode()
    err = rel_l2(o, ro)
    log(f"  {label}: rel-L2 {err:.3e} (bound {TOL['bf16']}), max abs {np.abs(o - ro).max():.3e}")
    assert np.all(np.isfinite(o))
    assert err <= TOL["bf16"]
    B, H = p.q_nope.shape[:2]
    for b in range(B):
        if p.seq_len[b] > 0:
            assert rel_l2(o[b], ro[b]) <= TOL["bf16"], b
    check_lse(lse, rl, view, [(b, h) for b in range(B) for h in range(H) if p.seq_len[b] > 0], "bf16")


@pytest.mark.parametrize("H", [128, 256])
def test_h32_small_all_outputs(H):
    p = _problem([1, 33, 200, 1000, 64], H=H)
    log(f"[h32 small] H={H} lengths={p.seq_len.tolist()}")
    o, lse = DeviceProblem(p).step(poison=True)
    _check_all(p, o, lse, f"H={H}")


@pytest.mark.parametrize("name", ["v2_bf16", "long_bf16"])
def test_h32_full_size_sampled(name):
    wl = W.WORKLOADS[name]
    p = W.make_problem(wl)
    log(f"[h32 full] {name} B={wl.B} T={p.T}")
    o, lse = DeviceProblem(p).step(poison=True)
    assert np.all(np.isfinite(o))
    B = wl.B
    seqs = sorted({0, B - 1, int(np.argmax(p.seq_len)), int(np.argmin(p.seq_len))})
    heads = range(wl.H) if name == "v2_bf16" else [0, 31, 32, 64, 100, 127]
    pairs = [(b, h) for b in seqs for h in heads]
    view = OracleView(p)
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    err = rel_l2(got, ro)
    log(f"  {len(pairs)} (sequence, head) pairs: rel-L2 {err:.3e}")
    assert err <= TOL["bf16"]
    check_lse(np.array([lse[b, h] for b, h in pairs]), rl, view, pairs, "bf16")


def test_h32_empty_sequences_between_others():
    lengths = [0, 0, 1, 0, 32, 0, 0, 33, 64, 0, 1, 0]
    p = _problem([max(n, 1) for n in lengths], seed=5)
    dp = DeviceProblem(p)
    dp.seq_len.copy_(torch.tensor(lengths, dtype=torch.int32))
    log(f"[h32 gappy] lengths={lengths}")
    dp.decode(poison=True)
    torch.cuda.synchronize()
    o = dp.out.double().cpu().numpy()
    lse = dp.lse.double().cpu().numpy()
    empty = [b for b, n in enumerate(lengths) if n == 0]
    full = [b for b, n in enumerate(lengths) if n > 0]
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    p2 = _problem([max(n, 1) for n in lengths], seed=5)
    p2.seq_len = np.array(lengths, dtype=np.int32)
    view = OracleView(p2, apply_append=False)
    pairs = [(b, h) for b in full for h in range(128)]
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    assert rel_l2(got, ro) <= TOL["bf16"]
    check_lse(np.array([lse[b, h] for b, h in pairs]), rl, view, pairs, "bf16")


def test_h32_repeatable_and_paged_equals_contiguous():
    from tests.test_gpu_paged import _page
    p = _problem([1, 33, 200, 1000, 517], seed=9)
    dp = DeviceProblem(p)
    o1, l1 = dp.step(poison=True)
    o2, l2 = dp.step(poison=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    pc = _page(dp, 64, seed=1)
    dp.out.fill_(float("nan"))
    ws = dp.mla.alloc_workspace(pc, dp.H, dp.q_nope.dtype)
    dp.mla.mla_decode_paged(pc, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                            1.0 / math.sqrt(192.0), dp.out, dp.lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(dp.out.double().cpu().numpy(), o1)


def test_h32_agrees_with_pair_kernel(monkeypatch):
    p = _problem([200, 1000, 3000], seed=2)
    dp = DeviceProblem(p)
    oh, _ = dp.step()
    monkeypatch.delenv("MLA_H32")
    op, _ = dp.step()
    d = rel_l2(oh, op)
    log(f"[h32 vs pair] rel-L2 between the kernels {d:.3e}")
    assert d <= 1e-2
