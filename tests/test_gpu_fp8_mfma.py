"""GPU parity of the fp8-cache decode with the value contraction on fp8 MFMA
(MLA_FP8_MFMA=1: e4m3 value weights), against the fp64 oracle on the same
dequantised cache, at the fp8 bound (rel-L2 4e-2 on o).

The variant rounds each value weight p_t * scale_t to e4m3 (3 mantissa
bits), so its error is larger than the default path's; each test logs the
achieved rel-L2. Cases: every output of small ragged problems at 32, 64 and
128 heads (the three pair-kernel widths), the benchmark's full size
(sampled sequences, every head), row scales that jump by 2^6 inside a
sequence (the weight exponent moves down mid-segment and o is rescaled),
empty sequences between others, and a paged cache."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.problem import OracleView
from tests.gpu_util import TOL, DeviceProblem, check_lse, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def fp8_mfma(monkeypatch):
    monkeypatch.setenv("MLA_FP8_MFMA", "1")


def _problem(lengths, H, seed=None):
    wl = W.WORKLOADS["fp8_cache"]
    lengths = np.array(lengths)
    return W.make_problem(wl, seed=seed, B=len(lengths), lengths=lengths, H=H)


def _check_all(p, o, lse, label):
    view = OracleView(p)
    ro, rl = view.decode()
    err = rel_l2(o, ro)
    log(f"  {label}: rel-L2 {err:.3e} (bound {TOL['fp8']}), max abs {np.abs(o - ro).max():.3e}")
    assert np.all(np.isfinite(o))
    assert err <= TOL["fp8"]
    B, H = p.q_nope.shape[:2]
    for b in range(B):
        if p.seq_len[b] > 0:
            assert rel_l2(o[b], ro[b]) <= TOL["fp8"], b
    check_lse(lse, rl, view, [(b, h) for b in range(B) for h in range(H) if p.seq_len[b] > 0], "fp8")
    return err


@pytest.mark.parametrize("H", [32, 64, 128])
def test_fp8_mfma_small_all_outputs(H):
    p = _problem([1, 33, 200, 1000], H)
    log(f"[fp8 mfma small] H={H} lengths={p.seq_len.tolist()}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    _check_all(p, o, lse, f"H={H}")


def test_fp8_mfma_full_size_sampled():
    wl = W.WORKLOADS["fp8_cache"]
    p = W.make_problem(wl)
    log(f"[fp8 mfma full] B={wl.B} H={wl.H} T={p.T}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    assert np.all(np.isfinite(o))
    B = wl.B
    rng = np.random.default_rng(11)
    seqs = sorted({0, B - 1, int(np.argmax(p.seq_len)), int(np.argmin(p.seq_len)),
                   *[int(b) for b in rng.choice(B, 4, replace=False)]})
    pairs = [(b, h) for b in seqs for h in range(wl.H)]
    view = OracleView(p)
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    err = rel_l2(got, ro)
    log(f"  {len(seqs)} sequences, every head: pooled rel-L2 {err:.3e} (bound {TOL['fp8']})")
    assert err <= TOL["fp8"]
    for b in seqs:
        idx = [i for i, (bb, _) in enumerate(pairs) if bb == b]
        assert rel_l2(got[idx], ro[idx]) <= TOL["fp8"], b
    check_lse(np.array([lse[b, h] for b, h in pairs]), rl, view, pairs, "fp8")


def test_fp8_mfma_scale_jumps_inside_a_sequence():
    """Rows 700.. of the long sequence get 64x larger scales (and rows
    300..339 64x smaller): the first tile past 700 lowers the weight
    exponent and rescales what the segment has accumulated."""
    p = _problem([1500, 90, 700], 128, seed=5)
    s0 = int(p.seq_start[0])
    scale = p.row_scale.numpy().copy()
    scale[s0 + 700:s0 + 1500] *= 64.0
    scale[s0 + 300:s0 + 340] /= 64.0
    p.row_scale = torch.from_numpy(scale)
    log("[fp8 mfma scale jumps] lengths=[1500, 90, 700]")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    _check_all(p, o, lse, "scale jumps")


def test_fp8_mfma_empty_sequences_between_others():
    lengths = [0, 257, 0, 0, 31, 0]
    p = _problem([max(n, 1) for n in lengths], 128, seed=3)
    dp = DeviceProblem(p)
    dp.seq_len.copy_(torch.tensor(lengths, dtype=torch.int32))
    log(f"[fp8 mfma empty] lengths={lengths}")
    dp.decode(poison=True)
    torch.cuda.synchronize()
    o = dp.out.double().cpu().numpy()
    lse = dp.lse.double().cpu().numpy()
    empty = [b for b, n in enumerate(lengths) if n == 0]
    full = [b for b, n in enumerate(lengths) if n > 0]
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    p2 = _problem([max(n, 1) for n in lengths], 128, seed=3)
    p2.seq_len = np.array(lengths, dtype=np.int32)
    view = OracleView(p2, apply_append=False)
    pairs = [(b, h) for b in full for h in range(128)]
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    err = rel_l2(got, ro)
    log(f"  rel-L2 {err:.3e}")
    assert err <= TOL["fp8"]
    check_lse(np.array([lse[b, h] for b, h in pairs]), rl, view, pairs, "fp8")


def test_fp8_mfma_paged_equals_contiguous():
    from tests.test_gpu_paged import _page
    p = _problem([1, 33, 200, 1000, 517], 128, seed=9)
    dp = DeviceProblem(p)
    o, _ = dp.step(poison=True)
    pc = _page(dp, 64, seed=1)
    dp.out.fill_(float("nan"))
    ws = dp.mla.alloc_workspace(pc, dp.H, dp.q_nope.dtype)
    dp.mla.mla_decode_paged(pc, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                            1.0 / math.sqrt(192.0), dp.out, dp.lse, ws)
    torch.cuda.synchronize()
    op = dp.out.to(torch.float64).cpu().numpy()
    log(f"[fp8 mfma paged] max |paged - contiguous| {np.abs(op - o).max():.3e}")
    assert np.array_equal(op, o)


def test_fp8_mfma_differs_from_default_path_only_by_weight_rounding(monkeypatch):
    """The same problem with MLA_FP8_MFMA unset runs the widened path; the
    two agree to the weight-rounding error and are not bitwise equal (so the
    switch really selects the fp8-MFMA kernel)."""
    p = _problem([200, 1000], 128, seed=2)
    dp = DeviceProblem(p)
    o8, _ = dp.step()
    monkeypatch.delenv("MLA_FP8_MFMA")
    ob, _ = dp.step()
    d = rel_l2(o8, ob)
    log(f"[fp8 mfma vs widened] rel-L2 between the paths {d:.3e}")
    assert 0 < d <= TOL["fp8"]
