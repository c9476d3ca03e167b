"""MLA_DEBUG=1: the entry points check the device-resident contract (lengths
in [1, capacity], appended tokens' sequence and position in range, rows
inside the cache) before launching and report a violation as
MLA_ERR_INVALID_ARGUMENT; without it the same values are clamped or skipped."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import DeviceProblem

pytestmark = pytest.mark.gpu


def _problem():
    p = W.make_problem(W.WORKLOADS["v2lite_bf16"], seed=3, B=3, lengths=np.array([5, 40, 9]))
    return DeviceProblem(p)


def _decode(dp):
    dp.mla.mla_decode(dp.cache, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                      1.0 / math.sqrt(192.0), dp.out, dp.lse, dp.ws)
    torch.cuda.synchronize()


def _append_absorb(dp):
    dp.mla.mla_append_absorb(dp.cache, dp.h, dp.w_dkv, dp.w_kr, dp.tok_seq, dp.tok_pos,
                             dp.p.wl.rope_base, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk,
                             dp.w_uv, 1.0 / math.sqrt(192.0), dp.out, dp.lse, dp.ws)
    torch.cuda.synchronize()


def _invalid(fn, dp):
    with pytest.raises(dp.mla.MlaError) as e:
        fn(dp)
    assert e.value.status == dp.mla.MLA_ERR_INVALID_ARGUMENT


def test_debug_mode_reports_contract_violations(monkeypatch):
    dp = _problem()
    dp.append()
    _decode(dp)
    ref = dp.out.clone()
    cap = dp.cache.seq_capacity.cpu().numpy()

    monkeypatch.setenv("MLA_DEBUG", "1")
    # a valid call runs and gives the same result
    dp.out.zero_()
    _decode(dp)
    assert torch.equal(dp.out, ref)
    dp.append()
    _append_absorb(dp)

    good = dp.seq_len.clone()
    for bad in (0, int(cap[1]) + 1, -3):
        dp.seq_len.copy_(good)
        dp.seq_len[1] = bad
        _invalid(_decode, dp)
        _invalid(_append_absorb, dp)
    dp.seq_len.copy_(good)

    good_pos, good_seq = dp.tok_pos.clone(), dp.tok_seq.clone()
    dp.tok_pos[0] = int(cap[int(good_seq[0])])            # one past the capacity
    _invalid(lambda d: d.append(), dp)
    _invalid(_append_absorb, dp)
    dp.tok_pos.copy_(good_pos)
    dp.tok_seq[2] = dp.B                                   # no such sequence
    _invalid(lambda d: d.append(), dp)
    dp.tok_seq.copy_(good_seq)

    # without the variable the same out-of-contract length is clamped
    monkeypatch.delenv("MLA_DEBUG")
    dp.seq_len[1] = int(cap[1]) + 1
    _decode(dp)
    assert torch.isfinite(dp.out.float()).all()
