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
        assert p.rows.shape == (p.total_rows, 576)
        assert p.q_nope.shape == (2, 16, 128) and p.q_pe.shape == (2, 16, 64)
        assert p.w_uk.shape == (16, 128, 512) and p.w_uv.shape == (16, 512, 128)
        assert np.all(p.seq_capacity >= p.seq_len)
        assert p.seq_start[1] == p.seq_capacity[0]
        assert (p.row_scale is not None) == (wl.cache == "fp8")
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
