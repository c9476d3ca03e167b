"""Parity over a fixed set of randomly drawn shapes: batch sizes, head counts,
cache dtypes and length mixes (short, long, empty, single-token sequences)
that exercise the work split's corner cases (workers with no tiles, ranges
crossing several sequences, one- and many-slot rows) and every merge + W_UV
launch. Sampled (sequence, head) outputs and lse against the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from oracle.problem import OracleView
from tests.gpu_util import TOL, DeviceProblem, check_lse, log, rel_l2

pytestmark = pytest.mark.gpu

BASE = {"bf16": "v2_bf16", "fp8": "fp8_cache", "f32": "tiny_fp32"}


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    cache = ["bf16", "bf16", "fp8", "f32"][seed % 4]
    H = int(rng.choice([16, 32, 64, 128])) if cache != "f32" else int(rng.choice([16, 32]))
    B = int(rng.choice([1, 3, 8, 17, 40, 96, 200]))
    mix = seed % 3
    if mix == 0:
        lengths = rng.integers(1, 64, size=B)                  # mostly one- or two-tile rows
    elif mix == 1:
        lengths = rng.integers(1, 3000, size=B)                # several tiles, ragged tails
    else:
        lengths = np.where(rng.random(B) < 0.3, 0, rng.integers(1, 900, size=B))  # with empties
        lengths[0] = max(int(lengths[0]), 1)
    return cache, H, B, lengths


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes(seed):
    cache, H, B, lengths = _case(seed)
    p = W.make_problem(W.WORKLOADS[BASE[cache]], seed=seed, B=B, lengths=lengths, H=H)
    log(f"[sweep {seed}] cache={cache} B={B} H={H} T={p.T}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    rng = np.random.default_rng(seed)
    live = [b for b in range(B) if lengths[b] > 0]
    pairs = sorted({(int(rng.choice(live)), int(rng.integers(H))) for _ in range(20)})
    view = OracleView(p)
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    gl = np.array([lse[b, h] for b, h in pairs])
    err = rel_l2(got, ro)
    log(f"  rel-L2 {err:.3e} max abs {np.abs(got - ro).max():.3e}")
    assert err <= TOL[cache]
    check_lse(gl, rl, view, pairs, cache)
    # empty sequences: zero output, lse = -inf
    for b in range(B):
        if lengths[b] == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
