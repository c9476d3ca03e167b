"""Pins of the oracle's prefill (causal multi-query attention) against what
the definition fixes: the first position attends one row (closed form), a
brute-force loop on a tiny case, causality (rows after a query's position
do not move it, rows before do), every query equals a decode over its
prefix (the decode oracle is pinned on its own), and the positions of a
chunk."""
import math

import numpy as np
import pytest

import oracle
from oracle import mla
import workloads as W
from oracle.problem import PrefillOracleView


def _rand(rng, L, n_heads=2):
    C = rng.standard_normal((L, 512))
    R = rng.standard_normal((L, 64))
    w_uk = rng.standard_normal((n_heads, 128, 512)) / math.sqrt(512)
    w_uv = rng.standard_normal((n_heads, 512, 128)) / math.sqrt(512)
    return C, R, w_uk, w_uv


def test_first_position_attends_one_row():
    rng = np.random.default_rng(0)
    C, R, w_uk, w_uv = _rand(rng, 7)
    qn = rng.standard_normal((3, 128))
    qp = rng.standard_normal((3, 64))
    o, lse = oracle.prefill_head(C, R, qn, qp, w_uk[1], w_uv[1], np.array([0, 0, 0]))
    v0 = np.array([sum(C[0, j] * w_uv[1, j, i] for j in range(512)) for i in range(128)])
    k0 = np.array([sum(w_uk[1, i, j] * C[0, j] for j in range(512)) for i in range(128)])
    for n in range(3):
        assert np.allclose(o[n], v0, rtol=1e-12, atol=1e-12)
        s00 = (qn[n] @ k0 + qp[n] @ R[0]) / math.sqrt(192.0)
        assert math.isclose(lse[n], s00, rel_tol=1e-12, abs_tol=1e-12)


def test_brute_force_tiny():
    """Three rows, every position a query, one head: K, V, scores, the
    causal softmax and the output as explicit loops."""
    rng = np.random.default_rng(1)
    L = 3
    C, R, w_uk, w_uv = _rand(rng, L, 1)
    qn = rng.standard_normal((L, 128))
    qp = rng.standard_normal((L, 64))
    K = [[sum(w_uk[0, i, j] * C[t, j] for j in range(512)) for i in range(128)] for t in range(L)]
    V = [[sum(C[t, j] * w_uv[0, j, i] for j in range(512)) for i in range(128)] for t in range(L)]
    o, lse = oracle.prefill_head(C, R, qn, qp, w_uk[0], w_uv[0], np.arange(L))
    for q in range(L):
        s = []
        for t in range(q + 1):
            dot = sum(qn[q, i] * K[t][i] for i in range(128)) + sum(qp[q, i] * R[t, i] for i in range(64))
            s.append(dot / math.sqrt(192.0))
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        ref = [sum(e[t] / z * V[t][i] for t in range(q + 1)) for i in range(128)]
        assert np.allclose(o[q], ref, rtol=1e-10, atol=1e-12), q
        assert math.isclose(lse[q], m + math.log(z), rel_tol=1e-12, abs_tol=1e-12)


def test_rows_after_a_query_do_not_move_it():
    rng = np.random.default_rng(2)
    L = 40
    C, R, w_uk, w_uv = _rand(rng, L)
    pos = np.array([3, 10, 25, 39])
    qn = rng.standard_normal((4, 128))
    qp = rng.standard_normal((4, 64))
    o, lse = oracle.prefill_head(C, R, qn, qp, w_uk[0], w_uv[0], pos)
    C2, R2 = C.copy(), R.copy()
    C2[11:] += 5.0
    R2[11:] -= 3.0
    o2, lse2 = oracle.prefill_head(C2, R2, qn, qp, w_uk[0], w_uv[0], pos)
    assert np.array_equal(o[:2], o2[:2]) and np.array_equal(lse[:2], lse2[:2])
    assert not np.allclose(o[2:], o2[2:])
    C3 = C.copy()
    C3[3] += 1.0                               # a row every query sees
    o3, _ = oracle.prefill_head(C3, R, qn, qp, w_uk[0], w_uv[0], pos)
    assert all(not np.allclose(o[i], o3[i]) for i in range(4))


def test_every_query_is_a_decode_over_its_prefix():
    rng = np.random.default_rng(3)
    L = 50
    C, R, w_uk, w_uv = _rand(rng, L)
    pos = np.arange(L - 20, L)
    qn = rng.standard_normal((20, 128))
    qp = rng.standard_normal((20, 64))
    for h in range(2):
        o, lse = oracle.prefill_head(C, R, qn, qp, w_uk[h], w_uv[h], pos)
        for i, p in enumerate(pos):
            od, ld = oracle.decode_head(C[:p + 1], R[:p + 1], qn[i], qp[i], w_uk[h], w_uv[h])
            assert np.allclose(o[i], od, rtol=1e-12, atol=1e-13), (h, i)
            assert math.isclose(lse[i], ld, rel_tol=1e-12)


def test_chunk_positions_are_the_last_slots():
    assert oracle.prefill_positions(10, 3).tolist() == [7, 8, 9]
    assert oracle.prefill_positions(4, 4).tolist() == [0, 1, 2, 3]
    assert oracle.prefill_positions(5, 0).tolist() == []
    with pytest.raises(ValueError):
        oracle.prefill_positions(3, 4)


def test_problem_view_splits_queries_by_sequence():
    """prefill_problem puts sequence b's queries at rows q_start[b].. and
    its positions at the end of b; a sequence with no queries is skipped;
    heads left out stay 0 / -inf."""
    wl = W.PREFILL_WORKLOADS["prefill_bf16"]
    p = W.make_prefill_problem(wl, lengths=[6, 9, 4], n_queries=[2, 0, 4], H=3)
    view = PrefillOracleView(p)
    o, lse = view.prefill(heads=[0, 2])
    assert o.shape == (6, 3, 128) and lse.shape == (6, 3)
    assert np.all(o[:, 1] == 0) and np.all(np.isneginf(lse[:, 1]))
    rows0, rows2 = view.rows64(0), view.rows64(2)
    for h in (0, 2):
        # sequence 0: queries at positions 4, 5; sequence 2: positions 0..3
        for qi, (rows, pos) in enumerate([(rows0, 4), (rows0, 5), (rows2, 0), (rows2, 1), (rows2, 2), (rows2, 3)]):
            od, ld = oracle.decode_head(rows[:pos + 1, :512], rows[:pos + 1, 512:], view.q_nope[qi, h],
                                        view.q_pe[qi, h], view.w_uk[h], view.w_uv[h])
            assert np.allclose(o[qi, h], od, rtol=1e-12, atol=1e-13)
            assert math.isclose(lse[qi, h], ld, rel_tol=1e-12)
