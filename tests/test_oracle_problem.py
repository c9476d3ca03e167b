"""The oracle on whole synthetic problems: widening of stored rows, the
append substitution, sampled versus full decode, and workload shapes."""
import numpy as np
import torch

import workloads as W
from oracle.problem import OracleView
from oracle import mla


def test_workload_shapes_and_lengths():
    for wl in W.WORKLOADS.values():
        p = W.make_problem(wl, B=2, lengths=np.array([3, 5]), H=16)
        assert p.rows.shape == (p.total_rows, 464 if wl.cache == "fp6" else 576)
        assert p.q_nope.shape == (2, 16, 128) and p.q_pe.shape == (2, 16, 64)
        assert p.w_uk.shape == (16, 128, 512) and p.w_uv.shape == (16, 512, 128)
        assert np.all(p.seq_capacity >= p.seq_len)
        assert p.seq_start[1] == p.seq_capacity[0]
        assert (p.row_scale is not None) == (wl.cache == "fp8")
        if wl.cache == "fp6":
            assert p.rows.dtype == torch.uint8 and np.all(p.rows[:, 450:].numpy() == 0)
    # seeded: the same seed draws the same lengths and values
    a = W.make_problem(W.WORKLOADS["v2lite_bf16"], B=3)
    b = W.make_problem(W.WORKLOADS["v2lite_bf16"], B=3)
    assert np.array_equal(a.seq_len, b.seq_len) and torch.equal(a.q_nope, b.q_nope)
    assert np.all((a.seq_len >= 1024) & (a.seq_len <= 4096))


def test_fp8_widening_matches_torch_decode():
    p = W.make_problem(W.WORKLOADS["fp8_cache"], B=2, lengths=np.array([4, 6]), H=16)
    v = OracleView(p)
    for b in range(2):
        s, L = int(p.seq_start[b]), int(p.seq_len[b])
        lib = (p.rows[s:s + L].view(torch.float8_e4m3fn).to(torch.float64)
               * p.row_scale[s:s + L].to(torch.float64)[:, None]).numpy()
        assert np.array_equal(v.rows64(b), lib)


def test_append_substitution_and_sampled_decode():
    p = W.make_problem(W.WORKLOADS["v2lite_bf16"], B=3, lengths=np.array([5, 1, 9]), H=16)
    v = OracleView(p)
    stored, scale, deq = v.append_stored
    for n in range(3):
        b, pos = int(p.tok_seq[n]), int(p.tok_pos[n])
        assert pos == p.seq_len[b] - 1
        assert np.array_equal(v.rows64(b)[pos], deq[n])
    o, lse = v.decode()
    assert o.shape == (3, 16, 128) and lse.shape == (3, 16)
    pairs = [(2, 15), (0, 3), (1, 0)]
    os_, ls_ = v.decode(pairs)
    for n, (b, h) in enumerate(pairs):
        assert np.array_equal(os_[n], o[b, h]) and ls_[n] == lse[b, h]
    # sequence 1 has length 1: its output is W_UV^T of the appended latent
    for h in range(16):
        want = deq[1, :512] @ v.w_uv[h]
        assert np.allclose(o[1, h], want, rtol=1e-12, atol=1e-13)


def test_rows_beyond_length_are_not_read():
    p = W.make_problem(W.WORKLOADS["tiny_fp32"], B=2, lengths=np.array([7, 4]), H=16)
    v = OracleView(p)
    o1, _ = v.decode()
    rows = p.rows.clone()
    m = torch.from_numpy(W.canary_mask(p))
    p.rows[m] = 1e30      # poison the canary rows
    o2, _ = OracleView(p).decode()
    p.rows.copy_(rows)
    assert np.array_equal(o1, o2)


def _selection_problem(through: str):
    """B sequences x H heads where every (b, h) has its own one-hot query
    aimed at a distinct token t*(b, h) of its sequence, so that softmax puts
    all but ~1e-26 of the weight on that token and o[b, h] must equal row
    t*(b, h) of W_UV[h] (v = W_UV[h]^T c with c = e_t*): a query, W_UK or
    W_UV taken from the wrong sequence or head lands on another token or
    another head's weights.

    through = "rope": the score is carried by q_pe . k_pe with k_pe_t = e_t;
    through = "latent": by q_nope . (W_UK[h] c_t) with c_t = e_t and W_UK[h]
    a head-specific permutation (row (j + 7h) % 128 picks latent dim j)."""
    B, H, L = 3, 4, 12
    rng = np.random.default_rng(11)
    alpha = 60.0 / mla.softmax_scale()         # scaled winning score 60
    tstar = np.array([[(5 * b + 3 * h + 1) % L for h in range(H)] for b in range(B)])
    assert len({(b, int(tstar[b, h])) for b in range(B) for h in range(H)}) > B  # distinct targets
    rows = np.zeros((B, L, 576))
    for b in range(B):
        for t in range(L):
            if through == "rope":
                rows[b, t, 512 + t] = 1.0
                rows[b, t, :512] = rng.standard_normal(512)   # latent part carries no score
            else:
                rows[b, t, t] = 1.0
    q_nope = np.zeros((B, H, 128))
    q_pe = np.zeros((B, H, 64))
    w_uk = np.zeros((H, 128, 512))
    for h in range(H):
        for j in range(512):
            w_uk[h, (j + 7 * h) % 128, j] = 1.0 if through == "latent" else 0.0
    for b in range(B):
        for h in range(H):
            t = int(tstar[b, h])
            if through == "rope":
                q_pe[b, h, t] = alpha
            else:
                q_nope[b, h, (t + 7 * h) % 128] = alpha
    w_uv = rng.standard_normal((H, 512, 128)) / np.sqrt(512)
    return B, H, L, rows, q_nope, q_pe, w_uk, w_uv, tstar


def test_problem_decode_selects_each_sequence_and_head():
    """Pins the per-(b, h) choice of q_nope, q_pe, W_UK and W_UV in the
    problem-level decode (decode_problem / decode_sampled) against the
    closed-form one-hot limit: o[b, h] = W_UV[h]^T c_t*, lse = the winning
    score (+ ln(1 + (L-1) e^-60))."""
    for through in ("rope", "latent"):
        B, H, L, rows, q_nope, q_pe, w_uk, w_uv, tstar = _selection_problem(through)
        o, lse = mla.decode_problem(lambda b: rows[b], q_nope, q_pe, w_uk, w_uv, B, H)
        for b in range(B):
            for h in range(H):
                t = int(tstar[b, h])
                want = rows[b, t, :512] @ w_uv[h]
                assert np.allclose(o[b, h], want, rtol=0, atol=1e-13 * np.abs(want).max()), \
                    (through, b, h)
                assert abs(lse[b, h] - (60.0 + np.log1p((L - 1) * np.exp(-60.0)))) < 1e-12
        # the sampled form picks the same pairs in any order
        pairs = [(2, 1), (0, 3), (1, 2), (0, 0)]
        os_, ls_ = mla.decode_sampled(lambda b: rows[b], q_nope, q_pe, w_uk, w_uv, pairs)
        for n, (b, h) in enumerate(pairs):
            assert np.array_equal(os_[n], o[b, h]) and ls_[n] == lse[b, h]


def test_oracle_view_selects_sequence_rows():
    """OracleView.rows64 hands decode the rows of the right sequence: each
    sequence's rows are marked with its index, and L = 1 per head gives
    W_UV[h]^T of that sequence's own row."""
    p = W.make_problem(W.WORKLOADS["tiny_fp32"], B=3, lengths=np.array([1, 1, 1]), H=16)
    for b in range(3):
        p.rows[int(p.seq_start[b])] = float(b + 1)
    v = OracleView(p)
    o, _ = v.decode()
    for b in range(3):
        for h in (0, 15):
            want = np.full(512, float(b + 1)) @ v.w_uv[h]
            assert np.allclose(o[b, h], want, rtol=1e-13, atol=1e-13)


def test_fp6_view_unpacks_codes_and_block_scales():
    """OracleView's fp6 rows: element i of a row is the 6-bit field at bits
    6i .. 6i+5 of the row's first 432 bytes, times 2^(its block's scale code
    - 127), the scale codes being bytes 432..449; checked on a hand-made row."""
    p = W.make_problem(W.WORKLOADS["fp6_cache"], B=1, lengths=np.array([2]), H=16)
    row = np.zeros(464, dtype=np.uint8)
    row[0] = 0b001000          # element 0: code 8 = 1.0
    row[0] |= 0b01 << 6        # element 1: low two bits of code 0b011001 ...
    row[1] = 0b0110            # ... high four bits: code 25 = 4.5
    row[24] = 0b100001         # element 32 (block 1): code 33 = -0.125
    row[432:450] = 127
    row[433] = 125             # block 1 scaled by 1/4
    p.rows[0] = torch.from_numpy(row)
    r = OracleView(p).rows64(0)[0]
    assert r[0] == 1.0 and r[1] == 4.5 and r[32] == -0.125 / 4
    assert np.all(r[2:32] == 0) and np.all(r[33:] == 0)
