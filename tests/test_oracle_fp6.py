"""Pins of the oracle's ~6-bit cache format (microscaling FP6: e2m3 elements,
blocks of 32 with one e8m0 scale) against the format's published facts and
closed forms: the e2m3 value set (largest 7.5, smallest normal 1, largest
subnormal 0.875, smallest 0.125, spacing 1/8 below 2, 1/4 in [2, 4), 1/2 in
[4, 8)), round-to-nearest-even ties and saturation, the shared exponent that
puts a block's largest element in [4, 8), the little-endian 6-bit packing
on hand-made bit patterns, and the dequantised rows' error bound."""
import numpy as np
import pytest

import oracle


def test_e2m3_value_set():
    v = oracle.e2m3_value_table()
    assert len(v) == 32 and v[0] == 0.0
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 7.5 and v[1] == 0.125
    assert 1.0 in v and v[np.searchsorted(v, 1.0) - 1] == 0.875
    steps = np.diff(v)
    assert np.all(steps[v[:-1] < 2.0] == 0.125)
    assert np.all(steps[(v[:-1] >= 2.0) & (v[:-1] < 4.0)] == 0.25)
    assert np.all(steps[v[:-1] >= 4.0] == 0.5)
    # negative codes mirror the positive ones
    assert np.array_equal(oracle.e2m3_decode(np.arange(32, 64)), -v)


def test_e2m3_encode_ties_saturation_and_round_trip():
    enc = oracle.e2m3_encode
    assert enc(0.0625) == 0            # tie between 0 and 1/8: even code
    assert enc(0.1875) == 2            # tie between 1/8 and 1/4: even code (1/4)
    assert enc(2.125) == 16            # tie between 2 and 2.25: even code (2)
    assert enc(2.375) == 18            # tie between 2.25 and 2.5: even code (2.5)
    assert enc(0.1) == 1 and enc(0.24) == 2
    assert enc(7.75) == 31 and enc(1e9) == 31 and enc(-1e9) == 63
    assert enc(-0.0) == 32 and enc(0.0) == 0
    codes = np.arange(64)
    back = enc(oracle.e2m3_decode(codes))
    assert np.array_equal(back, codes)
    with pytest.raises(ValueError):
        enc(np.nan)


def test_block_exponent_puts_the_largest_element_in_4_to_8():
    x = oracle.mx_block_exponent
    assert x(5.0) == 0 and x(4.0) == 0 and x(7.99) == 0
    assert x(3.99) == -1 and x(8.0) == 1 and x(0.5) == -3
    assert x(0.0) == -127 and x(2.0 ** 200) == 127 and x(2.0 ** -200) == -127
    a = np.abs(np.random.default_rng(0).standard_normal(1000)) * 10.0 ** np.random.default_rng(1).uniform(-5, 5, 1000)
    r = a / np.ldexp(1.0, x(a))
    assert np.all((r >= 4) & (r < 8))


def test_pack6_bit_layout():
    p = oracle.pack6
    assert p(np.array([[1, 0, 0, 0]])).tolist() == [[1, 0, 0]]
    assert p(np.array([[0, 1, 0, 0]])).tolist() == [[64, 0, 0]]          # bit 6
    assert p(np.array([[0, 0, 1, 0]])).tolist() == [[0, 16, 0]]          # bit 12
    assert p(np.array([[0, 0, 0, 1]])).tolist() == [[0, 0, 4]]           # bit 18
    assert p(np.array([[63, 63, 63, 63]])).tolist() == [[255, 255, 255]]
    assert p(np.array([[0, 0, 0, 0, 5, 0, 0, 0]])).tolist() == [[0, 0, 0, 5, 0, 0]]
    c = np.random.default_rng(2).integers(0, 64, size=(5, 576))
    assert np.array_equal(oracle.unpack6(p(c)), c)
    assert p(c).shape == (5, 432)


def test_quantized_rows_within_half_a_step():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((40, 576)) * np.exp(rng.uniform(-3, 3, (40, 1)))
    rows[5, :32] = 0.0                                  # an all-zero block
    stored, none, deq = oracle.quantize_rows(rows, "fp6")
    assert none is None and stored.shape == (40, 464) and stored.dtype == np.uint8
    assert np.all(stored[:, 450:] == 0)
    scales = stored[:, 432:450]
    assert np.array_equal(oracle.fp6_rows(stored), deq)
    assert np.array_equal(oracle.unpack6(stored[:, :432]).reshape(40, 18, 32)[5, 0], np.zeros(32))
    assert np.all(deq[5, :32] == 0) and scales[5, 0] == 0
    X = scales.astype(np.int64) - 127
    q = np.repeat(np.ldexp(1.0, X), 32, axis=1)          # the block's unit
    mag = np.abs(rows) / q
    half_step = np.where(mag < 2, 1 / 16, np.where(mag < 4, 1 / 8, 1 / 4))
    err = np.abs(deq - rows) / q
    # elements rounded into [4, 8) stay within half a step, except those past
    # 7.75, which saturate to 7.5 (less than half of the unit 1 beyond)
    ok = (err <= half_step + 1e-12) | ((mag > 7.75) & (err <= 0.5 + 1e-12))
    assert np.all(ok)
    # each block's largest element sits in [4, 8) of its unit before rounding
    bmax = mag.reshape(40, 18, 32).max(axis=2)
    assert np.all(((bmax >= 4) & (bmax < 8)) | (bmax == 0))
