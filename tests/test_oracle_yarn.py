"""Pins of the oracle's YaRN frequencies and softmax factor (discosf
explainer, "decoupled RoPE and YaRN" section: scale 40, alpha 1, beta 32,
160K target; the formula is the published YaRN method's). Each check rests on
what the method means, not on the oracle's own arithmetic: which pairs keep
their frequency, which are slowed by exactly the scale, the linear ramp
between, the closed form of the temperature, and RoPE's relative property."""
import math

import numpy as np
import pytest

import oracle

S, ALPHA, BETA, BASE = 40.0, 1.0, 32.0, 10000.0
L = 160 * 1024 // 40            # the original context: 160K target / scale 40 = 4096


def test_scale_one_is_plain_rope():
    f = oracle.yarn_inv_freq(BASE, 1.0, ALPHA, BETA, L)
    t = oracle.rope_inv_freq(BASE)
    assert np.allclose(f, t, rtol=1e-15, atol=0)


def test_which_pairs_are_kept_slowed_or_mixed():
    f = oracle.yarn_inv_freq(BASE, S, ALPHA, BETA, L)
    kept = slowed = mixed = 0
    for i in range(32):
        theta = BASE ** (-2.0 * i / 64)
        tokens_per_turn = 2 * math.pi / theta            # wavelength in tokens
        turns = L / tokens_per_turn                      # rotations over the original context
        if turns >= BETA:                                # fast pairs: unchanged
            assert f[i] == pytest.approx(theta, rel=1e-14)
            kept += 1
        elif turns <= ALPHA:                             # slow pairs: wavelength x40
            assert 2 * math.pi / f[i] == pytest.approx(S * tokens_per_turn, rel=1e-14)
            slowed += 1
        else:
            assert theta / S < f[i] < theta
            mixed += 1
    # with base 10000 and 64 dims the pages' constants give all three kinds
    assert kept == 11 and mixed == 12 and slowed == 9, (kept, mixed, slowed)
    # frequencies stay ordered: a later pair never turns faster
    assert np.all(np.diff(f) < 0)


def test_ramp_is_linear_in_turns():
    # choose the original context so that pair 10 turns exactly halfway
    # between alpha and beta: its frequency is the mean of theta/s and theta
    theta10 = BASE ** (-20.0 / 64)
    ctx = 0.5 * (ALPHA + BETA) * 2 * math.pi / theta10
    f = oracle.yarn_inv_freq(BASE, S, ALPHA, BETA, ctx)
    assert f[10] == pytest.approx(0.5 * (theta10 / S + theta10), rel=1e-14)
    # and a quarter of the way: three quarters of theta/s plus a quarter of theta
    ctx = (ALPHA + 0.25 * (BETA - ALPHA)) * 2 * math.pi / theta10
    f = oracle.yarn_inv_freq(BASE, S, ALPHA, BETA, ctx)
    assert f[10] == pytest.approx(0.75 * theta10 / S + 0.25 * theta10, rel=1e-14)


def test_softmax_factor_closed_forms():
    assert oracle.yarn_softmax_factor(math.exp(10.0)) == pytest.approx(4.0, rel=1e-14)   # (0.1*10+1)^2
    assert oracle.yarn_softmax_factor(1.0) == 1.0
    assert oracle.yarn_softmax_factor(0.5) == 1.0
    assert oracle.yarn_softmax_factor(math.exp(5.0)) == pytest.approx(2.25, rel=1e-14)   # 1.5^2


def test_yarn_rope_keeps_relative_position_property():
    rng = np.random.default_rng(3)
    f = oracle.yarn_inv_freq(BASE, S, ALPHA, BETA, L)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(0, 5), (17, 4096), (100000, 131071), (4095, 4097)]:
        lhs = oracle.rope_rotate(q, m, BASE, f) @ oracle.rope_rotate(k, n, BASE, f)
        rhs = q @ oracle.rope_rotate(k, n - m, BASE, f)
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)
    # position 0 is the identity; norms are kept
    assert np.array_equal(oracle.rope_rotate(k, 0, BASE, f), k)
    assert np.linalg.norm(oracle.rope_rotate(k, 123456, BASE, f)) == pytest.approx(np.linalg.norm(k), rel=1e-14)


def test_append_with_yarn_table_rotates_only_the_rope_part():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((3, 16))
    wd, wk = rng.standard_normal((512, 16)), rng.standard_normal((64, 16))
    pos = np.array([0, 4096, 131071])
    f = oracle.yarn_inv_freq(BASE, S, ALPHA, BETA, L)
    plain = oracle.append_rows_exact(h, wd, wk, pos, BASE)
    yarn = oracle.append_rows_exact(h, wd, wk, pos, BASE, f)
    assert np.array_equal(plain[:, :512], yarn[:, :512])       # c_KV is position-free
    assert np.array_equal(plain[0], yarn[0])                   # position 0: no rotation
    # the first 11 pairs turn at their original speed, the rest do not
    assert np.allclose(plain[:, 512:512 + 22], yarn[:, 512:512 + 22], rtol=1e-12, atol=1e-12)
    assert not np.allclose(plain[1:, 512 + 22:], yarn[1:, 512 + 22:])
