"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each checks a closed form, an
identity that a plausible mistake would break (dropped term, sign, index,
transposed operand), a printed value from the pages, or a library routine.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla
from oracle.numerics import (round_bf16, e4m3_decode, e4m3_encode, e4m3_value_table,
                             E4M3_MAX)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("="))
                out[k] = float(v)
    return out


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _tiny(rng, L, H=2):
    C = _rand(rng, L, 512)
    R = _rand(rng, L, 64)
    qn = _rand(rng, H, 128)
    qp = _rand(rng, H, 64)
    wuk = _rand(rng, H, 128, 512, std=1 / math.sqrt(512))
    wuv = _rand(rng, H, 512, 128, std=1 / math.sqrt(512))
    return C, R, qn, qp, wuk, wuv


def _rel(a, b):
    return float(np.linalg.norm(np.ravel(a - b)) / np.linalg.norm(np.ravel(b)))


# ---------------------------------------------------------------- cache sizes
def test_cache_size_worked_example_matches_printed_values():
    g = _golden("cache_size_worked_example.txt")
    per_tok = oracle.mla_cache_elements_per_token(int(g["d_c"]), int(g["d_r"]))
    assert per_tok == g["elements_per_token_per_layer"] == 576
    b1 = oracle.cache_bytes(int(g["context_tokens"]), int(g["layers"]), g["bits_per_element"])
    b64 = oracle.cache_bytes(int(g["context_tokens"]), int(g["layers"]), g["bits_per_element"],
                             batch=64)
    # printed to 2 and 3 significant figures
    assert round(b1 / 1e9, 1) == g["batch1_gb_printed"]
    assert round(b64 / 1e9) == g["batch64_gb_printed"]


def test_gqa_equivalence_pins_head_dim():
    g = _golden("cache_size_worked_example.txt")
    # 2.25 groups of GQA with d_h = 128 cache exactly the MLA row
    assert oracle.gqa_equivalent_groups(128) == g["gqa_groups_printed"]
    assert oracle.mha_cache_elements_per_token(2.25, 128) == 576


def test_mha_vs_mla_elements():
    assert oracle.mha_cache_elements_per_token(128, 128) == 32768
    assert oracle.mla_cache_elements_per_token() == 576
    assert oracle.mha_cache_elements_per_token(16, 128) == 4096
    # 98.24 % fewer elements per token than 128-head MHA with d_h = 128
    assert abs(1 - 576 / 32768 - 0.98242) < 1e-4


# ---------------------------------------------------------------- bf16 / fp8
def test_round_bf16_matches_torch_cast_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # fp32/bf16 subnormals
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -126, 0.0, -0.0],
                 dtype=np.float32),                                   # exact ties
    ])
    ours = round_bf16(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, lib)


def test_e4m3_decode_all_codes_closed_form_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    # closed form written from the bit fields, code by code
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert math.isnan(ours[c])
            continue
        v = (2.0 ** -6) * (m / 8) if e == 0 else (2.0 ** (e - 7)) * (1 + m / 8)
        assert ours[c] == (-v if s else v)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.nanmax(ours) == 448.0 and e4m3_value_table()[-1] == 448.0


def test_e4m3_encode_roundtrip_and_rounding():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    # in range, our RNE agrees with torch's cast (a library routine)
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * 60,
                        rng.standard_normal(5000) * 0.01,
                        np.array([0.0, 2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875, 440.0, 448.0])])
    x = x[np.abs(x) <= 448]
    x32 = x.astype(np.float32).astype(np.float64)
    ours = e4m3_decode(e4m3_encode(x32))
    lib = torch.from_numpy(x32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, lib)
    # saturation (torch's cast does not saturate, so this is checked by value)
    assert e4m3_decode(e4m3_encode(np.array([500.0, -1e9])))[0] == 448.0
    assert e4m3_decode(e4m3_encode(np.array([500.0, -1e9])))[1] == -448.0


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity_and_norm_preserved():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((5, 64))
    assert np.array_equal(mla.rope_rotate(k, np.zeros(5), 10000.0), k)
    pos = np.array([1, 7, 1000, 65535, 131071])
    r = mla.rope_rotate(k, pos, 10000.0)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(k, axis=1), rtol=1e-14)
    # pairwise norms preserved too (rotation acts on each (2i, 2i+1) pair)
    pn = lambda v: np.hypot(v[:, 0::2], v[:, 1::2])
    assert np.allclose(pn(r), pn(k), rtol=1e-13)


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    for m, n in [(0, 5), (3, 17), (1000, 1001), (5000, 70000)]:
        lhs = mla.rope_rotate(q, m, 10000.0) @ mla.rope_rotate(k, n, 10000.0)
        rhs = q @ mla.rope_rotate(k, n - m, 10000.0)
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(rhs))


def test_rope_unit_vector_angles_and_frequencies():
    # pair 0 turns by exactly pos radians (theta_0 = 1); pair 16 by pos/100
    # for base 10000 (theta_16 = 10000^(-1/2)); pairs are (2i, 2i+1)
    for pos in [0, 1, 3, 100, 4095, 131071]:
        e0 = np.zeros(64); e0[0] = 1
        r = mla.rope_rotate(e0, pos, 10000.0)
        ang = math.atan2(r[1], r[0])
        want = math.remainder(pos, 2 * math.pi)
        assert abs(ang - want) < 1e-9
        assert np.all(r[2:] == 0)
        e32 = np.zeros(64); e32[32] = 1
        r = mla.rope_rotate(e32, pos, 10000.0)
        assert abs(math.atan2(r[33], r[32]) - math.remainder(pos / 100.0, 2 * math.pi)) < 1e-9
    # the odd element of a pair rotates towards minus the even axis
    e1 = np.zeros(64); e1[1] = 1
    r = mla.rope_rotate(e1, math.pi / 2, 10000.0)
    assert abs(r[0] + 1) < 1e-15 and abs(r[1]) < 1e-15


# ---------------------------------------------------------------- append
def test_append_unit_hidden_picks_weight_columns():
    rng = np.random.default_rng(4)
    dm = 48
    wd = rng.standard_normal((512, dm))
    wk = rng.standard_normal((64, dm))
    for j in [0, 5, 47]:
        h = np.zeros((1, dm)); h[0, j] = 1
        rows = mla.append_rows_exact(h, wd, wk, np.array([9.0]), 10000.0)
        assert np.array_equal(rows[0, :512], wd[:, j])
        assert np.allclose(rows[0, 512:], mla.rope_rotate(wk[:, j], 9, 10000.0), rtol=0, atol=1e-15)
    # linearity in h
    h1, h2 = rng.standard_normal((1, dm)), rng.standard_normal((1, dm))
    p = np.array([33.0])
    a = mla.append_rows_exact(h1 + 2 * h2, wd, wk, p, 500.0)
    b = mla.append_rows_exact(h1, wd, wk, p, 500.0) + 2 * mla.append_rows_exact(h2, wd, wk, p, 500.0)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_quantize_rows_fp8_scale_and_bounds():
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((64, 576)) * rng.uniform(0.1, 10, size=(64, 1))
    rows[3] = 0.0
    codes, scale, deq = mla.quantize_rows(rows, "fp8")
    assert scale[3] == 1.0 and np.all(deq[3] == 0)
    amax = np.max(np.abs(rows), axis=1)
    nz = amax > 0
    assert np.allclose(scale[nz], amax[nz] / 448.0, rtol=2 ** -23)
    # the largest element lands on +-448 exactly
    i = np.argmax(np.abs(rows[nz]), axis=1)
    top = e4m3_decode(codes[nz][np.arange(nz.sum()), i])
    assert np.all(np.abs(top) == 448.0)
    # e4m3 relative error bound 2^-4 for normal codes; absolute 2^-10*scale below
    err = np.abs(deq - rows)
    bound = np.maximum(np.abs(rows) * 2 ** -4, 2 ** -10 * scale[:, None])
    assert np.all(err <= bound * (1 + 1e-12))


def test_quantize_rows_bf16_f32():
    x = np.array([[1 + 2 ** -9, 1 + 3 * 2 ** -9, 1 / 3]])
    v, _, d = mla.quantize_rows(x, "bf16")
    assert v[0, 0] == 1.0 and v[0, 1] == 1 + 2 ** -7
    v, _, _ = mla.quantize_rows(x, "f32")
    assert v[0, 2] == np.float32(1 / 3)


# ---------------------------------------------------------------- decode
def _absorbed(C, R, qn, qp, wuk, wuv):
    """The absorbed form (W_UK folded into the query, W_UV into the output)."""
    sig = 1 / math.sqrt(192)
    q_lat = wuk.T @ qn                      # [512]
    s = sig * (C @ q_lat + R @ qp)
    p = np.exp(s - s.max())
    p /= p.sum()
    return (p @ C) @ wuv


def test_absorbed_equals_unabsorbed():
    rng = np.random.default_rng(6)
    for L in [1, 2, 7, 33]:
        C, R, qn, qp, wuk, wuv = _tiny(rng, L)
        for h in range(2):
            o, _ = mla.decode_head(C, R, qn[h], qp[h], wuk[h], wuv[h])
            assert _rel(o, _absorbed(C, R, qn[h], qp[h], wuk[h], wuv[h])) < 1e-12


def test_transposed_weights_would_be_caught():
    # the absorbed identity distinguishes W_UK from its transpose-shaped misuse:
    # using W_UV where W_UK belongs changes the result
    rng = np.random.default_rng(7)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 9, H=1)
    o, _ = mla.decode_head(C, R, qn[0], qp[0], wuk[0], wuv[0])
    o_bad, _ = mla.decode_head(C, R, qn[0], qp[0], wuv[0].T, wuv[0])
    assert _rel(o_bad, o) > 1e-2


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(8)
    C, R, qn, qp, wuk, _ = _tiny(rng, 300)
    p = mla.attention_weights(C, R, qn[0], qp[0], wuk[0])
    assert np.all(p >= 0) and abs(p.sum() - 1) < 1e-13


def test_length_one_returns_wuv_of_the_token():
    rng = np.random.default_rng(9)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 1)
    for h in range(2):
        o, lse = mla.decode_head(C, R, qn[h], qp[h], wuk[h], wuv[h])
        want = np.array([sum(C[0, j] * wuv[h, j, i] for j in range(512)) for i in range(128)])
        assert np.allclose(o, want, rtol=1e-13, atol=1e-14)
        # lse of a single score is the score itself
        s = (sum(qn[h, i] * sum(wuk[h, i, j] * C[0, j] for j in range(512)) for i in range(128))
             + sum(qp[h, i] * R[0, i] for i in range(64))) / math.sqrt(192)
        assert abs(lse - s) < 1e-12


def test_zero_query_gives_uniform_average():
    rng = np.random.default_rng(10)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 17)
    o, lse = mla.decode_head(C, R, np.zeros(128), np.zeros(64), wuk[0], wuv[0])
    assert np.allclose(o, C.mean(axis=0) @ wuv[0], rtol=1e-13, atol=1e-14)
    assert abs(lse - math.log(17)) < 1e-13


def test_one_hot_limit_through_rope_key():
    # a query aligned with one token's RoPE key picks that token; this also
    # checks that q_pe meets the shared k_pe (a dropped RoPE term fails here)
    rng = np.random.default_rng(11)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 40)
    t = 23
    o, _ = mla.decode_head(C, R, np.zeros(128), 10 * R[t], wuk[0], wuv[0])
    assert np.allclose(o, C[t] @ wuv[0], rtol=1e-9, atol=1e-9)


def test_one_hot_limit_through_latent():
    # a query whose absorbed part aligns with one token's latent picks it;
    # checks that q_nope meets W_UK c (not c directly and not W_UK^T)
    rng = np.random.default_rng(12)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 40)
    t = 7
    q = 40 * (wuk[0] @ C[t]) / np.linalg.norm(wuk[0] @ C[t])
    o, _ = mla.decode_head(C, R, q, np.zeros(64), wuk[0], wuv[0])
    p = mla.attention_weights(C, R, q, np.zeros(64), wuk[0])
    assert p.argmax() == t and p[t] > 0.999
    assert np.allclose(o, C[t] @ wuv[0], rtol=2e-3, atol=2e-3)


def test_shift_invariance_through_shared_rope_key():
    # adding the same vector to every token's RoPE key shifts all scores of a
    # head by one constant; softmax output must not change, lse shifts
    rng = np.random.default_rng(13)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 25)
    v = rng.standard_normal(64)
    o1, l1 = mla.decode_head(C, R, qn[0], qp[0], wuk[0], wuv[0])
    o2, l2 = mla.decode_head(C, R + v, qn[0], qp[0], wuk[0], wuv[0])
    assert _rel(o2, o1) < 1e-12
    assert abs((l2 - l1) - (qp[0] @ v) / math.sqrt(192)) < 1e-10


def test_permutation_invariance_over_tokens():
    rng = np.random.default_rng(14)
    C, R, qn, qp, wuk, wuv = _tiny(rng, 50)
    perm = rng.permutation(50)
    o1, l1 = mla.decode_head(C, R, qn[1], qp[1], wuk[1], wuv[1])
    o2, l2 = mla.decode_head(C[perm], R[perm], qn[1], qp[1], wuk[1], wuv[1])
    assert _rel(o2, o1) < 1e-13 and abs(l1 - l2) < 1e-12
    # permuting only the RoPE keys (breaking the row pairing) changes it
    o3, _ = mla.decode_head(C, R[perm], qn[1], qp[1], wuk[1], wuv[1])
    assert _rel(o3, o1) > 1e-4


def test_oracle_error_vs_extended_precision_brute_force():
    # brute force in 80-bit long double, scalar loops over the definition
    rng = np.random.default_rng(15)
    L = 4
    C, R, qn, qp, wuk, wuv = _tiny(rng, L, H=1)
    o, lse = mla.decode_head(C, R, qn[0], qp[0], wuk[0], wuv[0])
    ld = np.longdouble
    Cl, Rl = C.astype(ld), R.astype(ld)
    K = np.array([[np.sum(wuk[0, i].astype(ld) * Cl[t]) for i in range(128)] for t in range(L)])
    V = np.array([[np.sum(Cl[t] * wuv[0, :, i].astype(ld)) for i in range(128)] for t in range(L)])
    sig = ld(1) / np.sqrt(ld(192))
    s = np.array([sig * (np.sum(K[t] * qn[0].astype(ld)) + np.sum(Rl[t] * qp[0].astype(ld)))
                  for t in range(L)])
    e = np.exp(s - s.max())
    p = e / e.sum()
    o_ld = np.array([np.sum(p * V[:, i]) for i in range(128)])
    assert float(np.linalg.norm((o - o_ld).astype(np.float64)) /
                 np.linalg.norm(o_ld.astype(np.float64))) < 1e-14
    assert abs(lse - float(s.max() + np.log(e.sum()))) < 1e-13


def test_empty_sequence_is_an_error():
    with pytest.raises(ValueError):
        mla.decode_head(np.zeros((0, 512)), np.zeros((0, 64)), np.zeros(128), np.zeros(64),
                        np.zeros((128, 512)), np.zeros((512, 128)))
