"""GPU parity of mla_decode (and mla_append where the workload has it)
against the fp64 oracle, through the C ABI.

Small cases run the oracle on every output; full-size cases (the workload
shapes the benchmark uses) compare sampled (sequence, head) outputs, which
the oracle computes one by one."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.problem import OracleView
from tests.gpu_util import TOL, DeviceProblem, check_lse, log, rel_l2

pytestmark = pytest.mark.gpu

SMALL_LENGTHS = {
    # ragged: 1 token, a partial tile, several tiles with a ragged tail
    16: [1, 37, 300, 64],
    128: [1, 33, 200],
}


def _small(name, lengths=None, seed=None):
    wl = W.WORKLOADS[name]
    lengths = np.array(lengths if lengths is not None else SMALL_LENGTHS[wl.H])
    return W.make_problem(wl, seed=seed, B=len(lengths), lengths=lengths)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_decode_small_all_outputs(name):
    p = _small(name)
    log(f"[decode small] {name} lengths={p.seq_len.tolist()} H={p.wl.H}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    view = OracleView(p)
    ro, rl = view.decode()
    err = rel_l2(o, ro)
    log(f"  rel-L2 {err:.3e} (bound {TOL[p.wl.cache]}), max abs {np.abs(o - ro).max():.3e}")
    assert np.all(np.isfinite(o))
    assert err <= TOL[p.wl.cache]
    B, H = p.q_nope.shape[:2]
    check_lse(lse, rl, view, [(b, h) for b in range(B) for h in range(H)], p.wl.cache)
    # every sequence on its own meets the bound too
    for b in range(p.q_nope.shape[0]):
        assert rel_l2(o[b], ro[b]) <= TOL[p.wl.cache], b


def _full_size_sequences(p, n_random):
    """First, last, longest and shortest sequence (the longest is split over
    the most workers), plus `n_random` others."""
    B = len(p.seq_len)
    pick = [0, B - 1, int(np.argmax(p.seq_len)), int(np.argmin(p.seq_len))]
    rng = np.random.default_rng(100 + p.wl.index)
    rest = [b for b in range(B) if b not in pick]
    pick += [int(b) for b in rng.choice(rest, size=min(n_random, len(rest)), replace=False)] if rest else []
    return sorted(set(pick))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_decode_full_size_all_heads(name):
    """At the benchmark's full size and launch configuration: every head of
    at least eight sequences (for the 128K workload, whose four sequences
    cost the oracle ~0.25 s per head each, every head of the first sequence
    and 16 heads of each other one), each sequence's rel-L2 and
    every lse checked, and the pooled rel-L2 and max-abs logged."""
    wl = W.WORKLOADS[name]
    p = W.make_problem(wl)
    log(f"[decode full] {name} B={wl.B} H={wl.H} T={p.T}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    assert np.all(np.isfinite(o))
    B, H = wl.B, wl.H
    if name == "long_bf16":
        rng = np.random.default_rng(7)
        pairs = [(0, h) for h in range(H)]
        pairs += [(b, int(h)) for b in range(1, B) for h in rng.choice(H, 16, replace=False)]
    else:
        pairs = [(b, h) for b in _full_size_sequences(p, 4) for h in range(H)]
    pairs = sorted(set(pairs))
    view = OracleView(p)
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    gl = np.array([lse[b, h] for b, h in pairs])
    err = rel_l2(got, ro)
    seqs = sorted({b for b, _ in pairs})
    log(f"  {len(seqs)} sequences, {len(pairs)} (b, h): pooled rel-L2 {err:.3e} "
        f"(bound {TOL[wl.cache]}), max abs {np.abs(got - ro).max():.3e}")
    assert err <= TOL[wl.cache]
    for b in seqs:
        idx = [i for i, (bb, _) in enumerate(pairs) if bb == b]
        e_b = rel_l2(got[idx], ro[idx])
        assert e_b <= TOL[wl.cache], (b, e_b)
    check_lse(gl, rl, view, pairs, wl.cache)


@pytest.mark.parametrize("name,lengths", [("v2lite_bf16", [700, 5, 1300]),
                                          ("v2_bf16", [3000, 5, 1300, 64]),
                                          ("fp8_cache", [900, 33, 2000]),
                                          ("fp6_cache", [900, 33, 2000])])
def test_decode_deterministic_and_repeatable(name, lengths):
    # no floating-point atomics: two runs over poisoned outputs and workspace
    # are bitwise equal, at 16 and at 128 heads (bf16 and fp8 caches)
    p = _small(name, lengths=lengths)
    dp = DeviceProblem(p)
    dp.decode(poison=True)
    a = dp.out.clone()
    la = dp.lse.clone()
    dp.decode(poison=True)
    assert torch.equal(a, dp.out) and torch.equal(la, dp.lse)


@pytest.mark.parametrize("name,lengths", [("v2lite_bf16", [700, 5, 1300]),
                                          ("v2_bf16", [3000, 5, 1300, 64]),
                                          ("v2_bf16", [40] * 300),
                                          ("fp8_cache", [900, 33, 2000]),
                                          ("tiny_fp32", [256, 3])])
def test_decode_without_lse(name, lengths):
    # lse = NULL takes its own branch in every merge kernel; out is bitwise
    # the same as with lse requested
    import head_latent_attention_14_amd as mla
    p = _small(name, lengths=lengths)
    dp = DeviceProblem(p)
    dp.decode(poison=True)
    torch.cuda.synchronize()
    ref = dp.out.clone()
    dp.out.fill_(float("nan"))
    dp.ws.fill_(0xFF)
    mla.mla_decode(dp.cache, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                   1.0 / math.sqrt(192.0), dp.out, None, dp.ws)
    torch.cuda.synchronize()
    assert torch.equal(ref, dp.out)


def test_nan_in_one_sequence_stays_there():
    p = _small("v2_bf16", lengths=[90, 150, 40])
    s1 = int(p.seq_start[1])
    p.rows[s1 + 17, 3] = float("nan")
    dp = DeviceProblem(p)
    o, _ = dp.step()
    assert np.all(np.isnan(o[1]))
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(o[2]))
    ro, _ = OracleView(p).decode([(0, h) for h in range(128)] + [(2, h) for h in range(128)])
    assert rel_l2(np.concatenate([o[0], o[2]]), ro) <= TOL["bf16"]


def test_canary_rows_poisoned_do_not_leak():
    # rows past each sequence's length hold huge values and NaN; output unchanged
    p = _small("v2lite_bf16", lengths=[33, 64, 2])
    mask = torch.from_numpy(W.canary_mask(p))
    p.rows[mask] = float("nan")
    dp = DeviceProblem(p)
    o, lse = dp.step()
    ro, rl = OracleView(p).decode()
    assert np.all(np.isfinite(o)) and rel_l2(o, ro) <= TOL["bf16"]


def test_zero_and_clamped_lengths():
    p = _small("v2lite_bf16", lengths=[5, 40, 9])
    dp = DeviceProblem(p)
    # sequence 0 gets length 0, sequence 2 asks for more rows than it owns
    dp.seq_len.copy_(torch.tensor([0, 40, 10_000], dtype=torch.int32))
    dp.decode(poison=True)
    torch.cuda.synchronize()
    o = dp.out.double().cpu().numpy()
    lse = dp.lse.double().cpu().numpy()
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    p2 = W.make_problem(W.WORKLOADS["v2lite_bf16"], B=3, lengths=np.array([5, 40, 9]))
    p2.seq_len = np.array([1, 40, int(p.seq_capacity[2])], dtype=np.int32)
    # no append ran on the device here, so the oracle must not apply it either
    ro, _ = OracleView(p2, apply_append=False).decode([(1, h) for h in range(16)] +
                                                     [(2, h) for h in range(16)])
    assert rel_l2(np.concatenate([o[1], o[2]]), ro) <= TOL["bf16"]


@pytest.mark.parametrize("B", [1, 17, 300, 1000])
def test_many_and_few_sequences(B):
    rng = np.random.default_rng(B)
    lengths = rng.integers(1, 200, size=B)
    p = W.make_problem(W.WORKLOADS["v2lite_bf16"], seed=B, B=B, lengths=lengths)
    log(f"[decode B={B}] T={p.T}")
    dp = DeviceProblem(p)
    o, _ = dp.step()
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(B, size=24), rng.integers(16, size=24))]
    ro, _ = OracleView(p).decode(sorted(set(pairs)))
    got = np.stack([o[b, h] for b, h in sorted(set(pairs))])
    assert rel_l2(got, ro) <= TOL["bf16"]


@pytest.mark.parametrize("B,H,maxlen", [(22, 16, 300), (500, 16, 300), (6, 128, 300), (300, 128, 40)])
def test_combine_row_blocks(B, H, maxlen):
    """Batches that reach the per-(head, row block) merge + W_UV launch with
    16-row blocks ending in 6 rows (one wave per row), 32-row blocks ending in
    20 rows (rows folded four at a time), 6 rows of 128 heads, and 300 short
    sequences of 128 heads (the split counts several tiles per sequence start
    there, so many workers' ranges hold no tile). Every row of the last block
    is checked, plus random ones, outputs and lse."""
    rng = np.random.default_rng(B * 1000 + H)
    lengths = rng.integers(1, maxlen, size=B)
    base = W.WORKLOADS["v2lite_bf16" if H == 16 else "v2_bf16"]
    p = W.make_problem(base, seed=B + H, B=B, lengths=lengths, H=H)
    log(f"[combine blocks] B={B} H={H} T={p.T}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    last = list(range(max(0, B - 20), B))
    pairs = {(b, int(h)) for b in last for h in rng.integers(H, size=2)}
    pairs |= {(int(b), int(h)) for b, h in zip(rng.integers(B, size=16), rng.integers(H, size=16))}
    pairs = sorted(pairs)
    view = OracleView(p)
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b, h in pairs])
    gl = np.array([lse[b, h] for b, h in pairs])
    assert rel_l2(got, ro) <= TOL["bf16"]
    check_lse(gl, rl, view, pairs, "bf16")


def test_other_head_counts():
    # 32 and 64 heads: one pair-kernel workgroup of 2 or 4 waves per worker;
    # 160 and 256 heads: several head groups per worker (5 x 32, 2 x 128)
    for H in [32, 64, 160, 256]:
        p = W.make_problem(W.WORKLOADS["v2_bf16"], B=2, lengths=np.array([77, 300]), H=H)
        dp = DeviceProblem(p)
        o, _ = dp.step()
        ro, _ = OracleView(p).decode()
        assert rel_l2(o, ro) <= TOL["bf16"], H


@pytest.mark.parametrize("H", [32, 64, 96, 128, 192])
def test_fp6_cache_pair_kernel_widths(H):
    # fp6 rows are widened tile by tile into bf16 in LDS inside the pair
    # kernel: 32, 64 and 128 heads per workgroup (96 heads: three 32-head
    # groups; 192: three 64-head groups); every output against the oracle on
    # the dequantised rows
    p = W.make_problem(W.WORKLOADS["fp6_cache"], B=4, lengths=np.array([1, 33, 200, 1000]), H=H)
    log(f"[fp6 pair] H={H} lengths={p.seq_len.tolist()}")
    dp = DeviceProblem(p)
    o, lse = dp.step(poison=True)
    view = OracleView(p)
    ro, rl = view.decode()
    err = rel_l2(o, ro)
    log(f"  rel-L2 {err:.3e} (bound {TOL['fp6']})")
    assert np.all(np.isfinite(o))
    assert err <= TOL["fp6"]
    for b in range(4):
        assert rel_l2(o[b], ro[b]) <= TOL["fp6"], b
    check_lse(lse, rl, view, [(b, h) for b in range(4) for h in range(H)], "fp6")


def test_prepared_calls_match_direct_calls():
    # the prepared binding marshals the same arguments once; results are bitwise equal
    import head_latent_attention_14_amd as mla
    p = _small("v2lite_bf16", lengths=[100, 37, 260])
    dp = DeviceProblem(p)
    o_direct, l_direct = dp.step()
    dp.out.zero_()
    dp.lse.zero_()
    pd = mla.PreparedDecode(dp.cache, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                            1.0 / math.sqrt(192.0), dp.out, dp.lse, dp.ws)
    pd.absorb()
    pd.attend()
    pd.combine()
    torch.cuda.synchronize()
    assert np.array_equal(dp.out.double().cpu().numpy(), o_direct)
    pd()
    torch.cuda.synchronize()
    assert np.array_equal(dp.out.double().cpu().numpy(), o_direct)
    assert np.array_equal(dp.lse.double().cpu().numpy(), l_direct)
    # stages 2 and 3 in one call
    dp.out.zero_()
    dp.lse.zero_()
    pd.absorb()
    pd.attend_combine()
    torch.cuda.synchronize()
    assert np.array_equal(dp.out.double().cpu().numpy(), o_direct)
    assert np.array_equal(dp.lse.double().cpu().numpy(), l_direct)


# Empty sequences between, before and after non-empty ones; lengths of 1, of a
# whole tile and one past it. Work is split in whole tiles, so these decide
# where workers start, where their segments end and which sequence follows.
GAPPY = [0, 0, 1, 0, 32, 0, 0, 33, 64, 0, 1, 0]


@pytest.mark.parametrize("name,H", [("v2lite_bf16", 16), ("v2_bf16", 32), ("v2_bf16", 128),
                                    ("fp8_cache", 16), ("fp8_cache", 128), ("fp6_cache", 16),
                                    ("fp6_cache", 128), ("tiny_fp32", 16)])
def test_empty_sequences_between_others(name, H):
    wl = W.WORKLOADS[name]
    make = np.array([max(n, 1) for n in GAPPY])
    p = W.make_problem(wl, seed=5, B=len(GAPPY), lengths=make, H=H)
    dp = DeviceProblem(p)
    dp.seq_len.copy_(torch.tensor(GAPPY, dtype=torch.int32))
    log(f"[decode gappy] {name} H={H} lengths={GAPPY}")
    dp.decode(poison=True)
    torch.cuda.synchronize()
    o = dp.out.double().cpu().numpy()
    lse = dp.lse.double().cpu().numpy()
    empty = [b for b, n in enumerate(GAPPY) if n == 0]
    full = [b for b, n in enumerate(GAPPY) if n > 0]
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    p2 = W.make_problem(wl, seed=5, B=len(GAPPY), lengths=make, H=H)
    p2.seq_len = np.array(GAPPY, dtype=np.int32)
    view = OracleView(p2, apply_append=False)
    pairs = [(b, h) for b in full for h in range(H)]
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b in full for h in range(H)])
    err = rel_l2(got, ro)
    log(f"  rel-L2 {err:.3e}")
    assert err <= TOL[wl.cache]
    gl = np.array([lse[b, h] for b in full for h in range(H)])
    check_lse(gl, rl, view, pairs, wl.cache)
    # every non-empty sequence on its own meets the bound too
    for i, b in enumerate(full):
        assert rel_l2(got[i * H:(i + 1) * H], ro[i * H:(i + 1) * H]) <= TOL[wl.cache], b


def _fused_step(dp, poison=True):
    import head_latent_attention_14_amd as mla
    if poison:
        dp.out.fill_(float("nan"))
        dp.lse.fill_(float("nan"))
        dp.ws.fill_(0xFF)
    scale = 1.0 / math.sqrt(192.0)
    mla.mla_append_absorb(dp.cache, dp.h, dp.w_dkv, dp.w_kr, dp.tok_seq, dp.tok_pos,
                          dp.p.wl.rope_base, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                          scale, dp.out, dp.lse, dp.ws)
    mla.mla_decode_attend(dp.cache, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv, scale,
                          dp.out, dp.lse, dp.ws)
    mla.mla_decode_combine(dp.cache, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv, scale,
                           dp.out, dp.lse, dp.ws)
    torch.cuda.synchronize()
    return (dp.out.double().cpu().numpy(), dp.lse.double().cpu().numpy(),
            dp.cache.rows.cpu().view(torch.int16).numpy().copy())


@pytest.mark.parametrize("full", [False, True])
def test_append_absorb_equals_append_then_decode(full):
    # one launch for append + absorb (bf16) gives bit-identical rows and outputs
    wl = W.WORKLOADS["v2lite_bf16"]
    p = W.make_problem(wl) if full else _small("v2lite_bf16")
    log(f"[append+absorb] full={full} B={p.q_nope.shape[0]}")
    a = DeviceProblem(p)
    o_ref, l_ref = a.step(poison=True)
    rows_ref = a.cache.rows.cpu().view(torch.int16).numpy().copy()
    b = DeviceProblem(p)
    o, l, rows = _fused_step(b)
    assert np.array_equal(rows, rows_ref)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(np.isnan(l), np.isnan(l_ref)) and np.array_equal(l[~np.isnan(l)],
                                                                            l_ref[~np.isnan(l_ref)])
    # and against the oracle (append applied)
    ro, _ = OracleView(p).decode([(0, 0), (p.q_nope.shape[0] - 1, 15)])
    assert rel_l2(np.stack([o[0, 0], o[-1, 15]]), ro) <= TOL["bf16"]


def test_append_absorb_two_launch_path():
    # a grid too large for one round of CUs (many heads, few tokens) takes
    # the two-launch path; results still match append then decode bitwise
    wl = W.WORKLOADS["v2lite_bf16"]
    p = W.make_problem(wl, B=40, lengths=np.arange(40) * 7 + 1, H=64)
    a = DeviceProblem(p)
    o_ref, _ = a.step(poison=True)
    rows_ref = a.cache.rows.cpu().view(torch.int16).numpy().copy()
    b = DeviceProblem(p)
    o, _, rows = _fused_step(b)
    assert np.array_equal(rows, rows_ref)
    assert np.array_equal(o, o_ref)


def test_append_absorb_paired_absorb_tiles():
    # 32 heads, 16 sequences: 36 append workgroups and 256 absorb tiles on
    # 219 workgroups, 37 of which run a second tile beside the first; rows
    # and outputs match append then decode bitwise, and the oracle
    wl = W.WORKLOADS["v2lite_bf16"]
    lengths = np.random.default_rng(32).integers(1, 700, size=16)
    p = W.make_problem(wl, seed=32, B=16, lengths=lengths, H=32)
    log(f"[append+absorb paired tiles] B=16 H=32 lengths={lengths.tolist()}")
    a = DeviceProblem(p)
    o_ref, _ = a.step(poison=True)
    rows_ref = a.cache.rows.cpu().view(torch.int16).numpy().copy()
    b = DeviceProblem(p)
    o, _, rows = _fused_step(b)
    assert np.array_equal(rows, rows_ref)
    assert np.array_equal(o, o_ref)
    pairs = [(0, 0), (7, 31), (15, 17)]
    ro, _ = OracleView(p).decode(pairs)
    assert rel_l2(np.stack([o[bb, hh] for bb, hh in pairs]), ro) <= TOL["bf16"]


def test_combine_fused_launch_all_outputs():
    # 64 short sequences at 16 heads: few slots per sequence, so the merge and
    # W_UV run as one launch; every output and lse against the oracle, with
    # two empty sequences among them
    rng = np.random.default_rng(64)
    lengths = rng.integers(1, 120, size=64)
    p = W.make_problem(W.WORKLOADS["v2lite_bf16"], seed=64, B=64, lengths=lengths)
    dp = DeviceProblem(p)
    lens = lengths.copy()
    lens[[5, 40]] = 0
    dp.seq_len.copy_(torch.from_numpy(lens.astype(np.int32)))
    dp.decode(poison=True)
    torch.cuda.synchronize()
    o = dp.out.double().cpu().numpy()
    lse = dp.lse.double().cpu().numpy()
    assert np.all(o[[5, 40]] == 0) and np.all(np.isneginf(lse[[5, 40]]))
    p2 = W.make_problem(W.WORKLOADS["v2lite_bf16"], seed=64, B=64, lengths=lengths)
    p2.seq_len = lens.astype(np.int32)
    full = [b for b in range(64) if lens[b] > 0]
    view = OracleView(p2, apply_append=False)
    pairs = [(b, h) for b in full for h in range(16)]
    ro, rl = view.decode(pairs)
    got = np.stack([o[b, h] for b in full for h in range(16)])
    assert rel_l2(got, ro) <= TOL["bf16"]
    gl = np.array([lse[b, h] for b in full for h in range(16)])
    check_lse(gl, rl, view, pairs, "bf16")


@pytest.mark.parametrize("name", ["fp8_cache", "tiny_fp32"])
def test_append_absorb_other_caches(name):
    # fp8 and f32 caches take the two-launch path of mla_append_absorb; rows,
    # row scales and outputs equal mla_append then mla_decode bitwise
    import head_latent_attention_14_amd as mla
    wl = W.WORKLOADS[name]
    lengths = np.array([3, 40, 97])
    p = W.make_problem(wl, seed=7, B=3, lengths=lengths)
    rng = np.random.default_rng(7)
    act = p.q_nope.dtype
    dm = 256
    h = torch.from_numpy(rng.standard_normal((3, dm)).astype(np.float32)).to(act).cuda()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) / 16).astype(np.float32)).to(act).cuda()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) / 16).astype(np.float32)).to(act).cuda()
    ts = torch.arange(3, dtype=torch.int32).cuda()
    tp = torch.from_numpy((lengths - 1).astype(np.int32)).cuda()
    scale = 1.0 / math.sqrt(192.0)
    res = []
    for fused in (False, True):
        dp = DeviceProblem(p)
        dp.out.fill_(float("nan"))
        dp.ws.fill_(0xFF)
        args = (dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv, scale, dp.out, dp.lse, dp.ws)
        if fused:
            mla.mla_append_absorb(dp.cache, h, wd, wk, ts, tp, 10000.0, *args)
            mla.mla_decode_attend(dp.cache, *args)
            mla.mla_decode_combine(dp.cache, *args)
        else:
            mla.mla_append(dp.cache, h, wd, wk, ts, tp, 10000.0)
            mla.mla_decode(dp.cache, *args)
        torch.cuda.synchronize()
        sc = dp.cache.row_scale.cpu().numpy().copy() if dp.cache.row_scale is not None else None
        res.append((dp.out.double().cpu().numpy(), _bits_of(dp.cache.rows), sc))
    (o0, r0, s0), (o1, r1, s1) = res
    assert np.array_equal(r0, r1)
    assert s0 is None or np.array_equal(s0, s1)
    assert np.array_equal(o0, o1) and np.all(np.isfinite(o1))


def _bits_of(t):
    t = t.cpu().contiguous()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]).numpy().copy()
