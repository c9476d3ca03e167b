"""GPU parity of mla_append against the oracle, through the C ABI.

RoPE indexing is checked exactly: with unit inputs the stored pair i of the
RoPE key is (cos(pos*theta_i), sin(pos*theta_i)), so its angle must equal
pos*theta_i reduced mod 2*pi (computed in fp64) to within 1e-6 rad, at
positions up to 131071; the written slot must be seq_start + pos and every
other row must keep its bytes."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import mla as omla
from oracle.numerics import e4m3_decode
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _mla():
    import head_latent_attention_14_amd as mla
    return mla


def _cache(dtype, caps, fill=None):
    mla = _mla()
    caps = np.asarray(caps, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]])
    total = int(caps.sum())
    if dtype == "fp8":
        rows = torch.randint(0, 0x7E, (total, 576), dtype=torch.uint8)
        scale = torch.rand(total) + 0.5
    elif dtype == "fp6":
        rows = torch.randint(0, 256, (total, 464), dtype=torch.uint8)
        scale = None
    else:
        rows = torch.randn(total, 576).to(W.TORCH_DTYPE[dtype])
        scale = None
    cache = mla.LatentCache(rows=rows.cuda(), seq_start=torch.from_numpy(starts).cuda(),
                            seq_capacity=torch.from_numpy(caps.astype(np.int32)).cuda(),
                            row_scale=scale.cuda() if scale is not None else None)
    return cache, starts


def _append(cache, h, wd, wk, seq, pos, base):
    mla = _mla()
    mla.mla_append(cache, h.cuda(), wd.cuda(), wk.cuda(),
                   torch.tensor(seq, dtype=torch.int32).cuda(),
                   torch.tensor(pos, dtype=torch.int32).cuda(), base)
    torch.cuda.synchronize()


def test_rope_indexing_exact_unit_probe():
    dm = 64
    positions = [0, 1, 2, 3, 100, 4095, 4096, 65535, 100000, 131071]
    n = len(positions)
    cache, starts = _cache("f32", [131072, 17])
    before = cache.rows.clone()
    h = torch.zeros(n, dm)
    h[:, 0] = 1.0
    wd = torch.zeros(512, dm)
    wd[7, 0] = 1.0                               # c_KV element 7 = 1 exactly
    wk = torch.zeros(64, dm)
    wk[0::2, 0] = 1.0                            # k = (1, 0, 1, 0, ...): every pair unit
    _append(cache, h, wd, wk, [0] * n, positions, 10000.0)
    rows = cache.rows.cpu().double().numpy()
    inv = omla.rope_inv_freq(10000.0)
    worst = 0.0
    for p in positions:
        r = rows[int(starts[0]) + p]
        assert r[7] == 1.0 and np.count_nonzero(r[:512]) == 1
        for i in range(32):
            ang = math.atan2(r[512 + 2 * i + 1], r[512 + 2 * i])
            want = math.remainder(p * float(inv[i]), 2 * math.pi)
            d = abs(math.remainder(ang - want, 2 * math.pi))
            worst = max(worst, d)
            assert d < 1e-6, (p, i, ang, want)
    log(f"  worst RoPE angle error {worst:.2e} rad")
    # only the addressed rows changed
    changed = np.nonzero(np.any(_bits(before) != _bits(cache.rows), axis=1))[0]
    assert sorted(changed.tolist()) == sorted(int(starts[0]) + p for p in positions)


def _bits(t):
    """Raw bits of a device tensor as a numpy integer array (any dtype)."""
    t = t.cpu().contiguous()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]).numpy()


def _dot_bound(h, wd, wk, pos, base):
    """Per-element bound on |fp32 result - exact|: the device accumulates
    products in fp32, so its error is at most a small multiple of
    2^-24 * sum_k |h_k w_k| (taken 2^-18 * S here, generous); the RoPE pair
    mixes two such sums."""
    ah, ad, ak = np.abs(h), np.abs(wd), np.abs(wk)
    S = np.concatenate([ah @ ad.T, ah @ ak.T], axis=1)
    pair = S[:, 512:].reshape(-1, 32, 2).sum(axis=2)
    S[:, 512:] = np.repeat(pair, 2, axis=1)
    return S * 2.0 ** -18


def _near_tie_bf16(x, bound):
    """True where the exact x lies within `bound` of a bf16 rounding midpoint."""
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    mid = (np.floor(np.abs(x) / ulp) + 0.5) * ulp
    return np.abs(np.abs(x) - mid) <= bound


@pytest.mark.parametrize("n_tok", [1, 5, 37, 64])
def test_append_bf16_values_and_slots(n_tok):
    rng = np.random.default_rng(n_tok)
    dm = 2048
    B = 8
    caps = rng.integers(40, 300, size=B)
    cache, starts = _cache("bf16", caps)
    before = cache.rows.clone()
    h = torch.from_numpy(rng.standard_normal((n_tok, dm)).astype(np.float32)).bfloat16()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    # distinct slots
    slots = rng.choice([(b, p) for b in range(B) for p in range(int(caps[b]))], size=n_tok,
                       replace=False)
    seq = [int(s[0]) for s in slots]
    pos = [int(s[1]) for s in slots]
    _append(cache, h, wd, wk, seq, pos, 10000.0)
    exact = omla.append_rows_exact(h.double().numpy(), wd.double().numpy(), wk.double().numpy(),
                                   np.array(pos, dtype=np.float64), 10000.0)
    stored, _, _ = omla.quantize_rows(exact, "bf16")
    rows = cache.rows.cpu().double().numpy()
    got = np.stack([rows[int(starts[s]) + p] for s, p in zip(seq, pos)])
    bound = _dot_bound(h.double().numpy(), wd.double().numpy(), wk.double().numpy(), pos,
                       10000.0)
    tie = _near_tie_bf16(exact, bound)
    mism = (got != stored) & ~tie
    log(f"  n_tok={n_tok}: {int((got != stored).sum())} of {got.size} differ, "
        f"{int(tie.sum())} near ties, {int(mism.sum())} off-tie mismatches")
    assert not mism.any()
    # near ties may land on either neighbour, never further than the fp32
    # accumulation error allows
    assert np.all(np.abs(got - exact) <= np.ldexp(1.0, np.frexp(exact)[1] - 8) + bound)
    changed = np.nonzero(np.any(_bits(before) != _bits(cache.rows), axis=1))[0]
    assert set(changed.tolist()) <= {int(starts[s]) + p for s, p in zip(seq, pos)}


def test_append_fp8_codes_and_scales():
    rng = np.random.default_rng(3)
    dm = 512
    n_tok = 40
    cache, starts = _cache("fp8", [64, 64])
    h = torch.from_numpy(rng.standard_normal((n_tok, dm)).astype(np.float32)).bfloat16()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) * rng.uniform(0.01, 0.2)).astype(np.float32)).bfloat16()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) * 0.05).astype(np.float32)).bfloat16()
    seq = [i % 2 for i in range(n_tok)]
    pos = [i // 2 for i in range(n_tok)]
    _append(cache, h, wd, wk, seq, pos, 10000.0)
    exact = omla.append_rows_exact(h.double().numpy(), wd.double().numpy(), wk.double().numpy(),
                                   np.array(pos, dtype=np.float64), 10000.0)
    codes_ref, scale_ref, deq_ref = omla.quantize_rows(exact, "fp8")
    rows = cache.rows.cpu().numpy()
    sc = cache.row_scale.cpu().double().numpy()
    idx = [int(starts[s]) + p for s, p in zip(seq, pos)]
    got_codes = rows[idx]
    got_scale = sc[idx]
    assert np.allclose(got_scale, scale_ref, rtol=1e-5, atol=0)
    got = e4m3_decode(got_codes) * got_scale[:, None]
    # a code may differ from the oracle's only where x/scale is near a rounding midpoint
    v = exact / scale_ref[:, None]
    _, e = np.frexp(np.abs(v))
    q = np.ldexp(1.0, np.maximum(e, -5) - 4)
    t = np.abs(v) / q
    tie = np.abs((t - np.floor(t)) - 0.5) < 0.02
    diff = e4m3_decode(got_codes) != e4m3_decode(codes_ref)
    log(f"  fp8 append: {int(diff.sum())} of {diff.size} codes differ ({int((diff & ~tie).sum())} off-tie)")
    assert not (diff & ~tie).any()
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert rel <= 4e-2


def test_append_fp6_codes_scales_and_padding():
    """fp6 append: every block's scale code and every element code equal the
    oracle's, except where the exact value lies within the fp32 accumulation
    error of a decision: a block maximum within 1e-5 (relative) of a power of
    two (the shared exponent), an element within 2% of a step of a rounding
    midpoint (the code); the padding bytes are zero."""
    rng = np.random.default_rng(4)
    dm = 512
    n_tok = 40
    cache, starts = _cache("fp6", [64, 64])
    h = torch.from_numpy(rng.standard_normal((n_tok, dm)).astype(np.float32)).bfloat16()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) * rng.uniform(0.01, 0.2)).astype(np.float32)).bfloat16()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) * 0.05).astype(np.float32)).bfloat16()
    seq = [i % 2 for i in range(n_tok)]
    pos = [i // 2 for i in range(n_tok)]
    _append(cache, h, wd, wk, seq, pos, 10000.0)
    exact = omla.append_rows_exact(h.double().numpy(), wd.double().numpy(), wk.double().numpy(),
                                   np.array(pos, dtype=np.float64), 10000.0)
    ref, _, deq_ref = omla.quantize_rows(exact, "fp6")
    idx = [int(starts[s]) + p for s, p in zip(seq, pos)]
    got = cache.rows.cpu().numpy()[idx]
    assert np.all(got[:, 450:] == 0)
    # shared exponents
    amax = np.abs(exact).reshape(n_tok, 18, 32).max(axis=2)
    near_pow2 = np.abs(np.log2(amax) - np.round(np.log2(amax))) < 1e-5
    sdiff = got[:, 432:450] != ref[:, 432:450]
    log(f"  fp6 append: {int(sdiff.sum())} of {sdiff.size} block scales differ")
    assert not (sdiff & ~near_pow2).any()
    # element codes, in blocks whose exponent agrees
    from oracle.numerics import unpack6
    gc, rc = unpack6(got[:, :432]), unpack6(ref[:, :432])
    X = np.repeat(ref[:, 432:450].astype(np.int64) - 127, 32, axis=1)
    mag = np.abs(exact) / np.ldexp(1.0, X)
    step = np.where(mag < 2, 1 / 8, np.where(mag < 4, 1 / 4, 1 / 2))
    frac = (mag / step) % 1.0
    tie = np.abs(frac - 0.5) < 0.02
    same_x = np.repeat(~sdiff, 32, axis=1)
    cdiff = (gc != rc) & same_x
    log(f"  fp6 append: {int(cdiff.sum())} of {cdiff.size} codes differ ({int((cdiff & ~tie).sum())} off-tie)")
    assert not (cdiff & ~tie).any()
    deq = omla.fp6_rows(got)
    err, err_ref = (np.linalg.norm(deq - exact), np.linalg.norm(deq_ref - exact))
    assert err <= 1.01 * err_ref + 1e-12


def test_append_skips_invalid_tokens():
    cache, starts = _cache("bf16", [10, 10])
    before = cache.rows.clone()
    dm = 64
    h = torch.randn(4, dm).bfloat16()
    wd = torch.randn(512, dm).bfloat16()
    wk = torch.randn(64, dm).bfloat16()
    # seq out of range, pos out of range (negative and >= capacity), one valid token
    _append(cache, h, wd, wk, [2, 0, 1, 1], [0, -1, 10, 3], 10000.0)
    changed = np.nonzero(np.any(_bits(before) != _bits(cache.rows), axis=1))[0]
    assert changed.tolist() == [int(starts[1]) + 3]


def test_append_then_decode_end_to_end_full_size():
    # the V2-Lite-shaped step: append one token per sequence, decode over it
    from oracle.problem import OracleView
    from tests.gpu_util import DeviceProblem, rel_l2
    p = W.make_problem(W.WORKLOADS["v2lite_bf16"])
    dp = DeviceProblem(p)
    o, _ = dp.step()
    view = OracleView(p)
    stored, _, _ = view.append_stored
    rows = dp.cache.rows.cpu().double().numpy()
    got = np.stack([rows[int(p.seq_start[b]) + int(p.tok_pos[b])] for b in range(p.wl.B)])
    assert rel_l2(got, stored) < 4e-3
    # the appended token is the last one of each sequence: check every head of 4 sequences
    pairs = [(b, h) for b in (0, 17, 40, 63) for h in range(16)]
    ro, _ = view.decode(pairs)
    assert rel_l2(np.stack([o[b, h] for b, h in pairs]), ro) <= 2e-2


@pytest.mark.parametrize("fused", [False, True])
def test_append_bf16_large_positions(fused):
    """The bf16 append kernels (mla_append's and the fused append + absorb
    launch) form the RoPE angle in fp64, reduce it there and take sine and
    cosine of the reduced angle in fp32: at positions up to 131071 the stored
    rows still equal the oracle's exact rows rounded to bf16, except where the
    exact value lies within the fp32 accumulation error of a rounding
    midpoint (an unreduced fp32 angle is off by up to ~5e-3 rad there, far
    outside that allowance)."""
    mla = _mla()
    rng = np.random.default_rng(131071)
    dm = 512
    positions = [0, 1, 4095, 4096, 32767, 65535, 100000, 131071] + \
        [int(x) for x in rng.integers(0, 131072, size=8)]
    n_tok = len(positions)
    caps = [131072, 131072]
    cache, starts = _cache("bf16", caps)
    before = cache.rows.clone()
    h = torch.from_numpy(rng.standard_normal((n_tok, dm)).astype(np.float32)).bfloat16()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    seq = [i % 2 for i in range(n_tok)]
    tseq = torch.tensor(seq, dtype=torch.int32).cuda()
    tpos = torch.tensor(positions, dtype=torch.int32).cuda()
    if fused:
        B, H = 2, 16
        seq_len = torch.tensor(caps, dtype=torch.int32).cuda()
        q_nope = torch.randn(B, H, 128).bfloat16().cuda()
        q_pe = torch.randn(B, H, 64).bfloat16().cuda()
        w_uk = (torch.randn(H, 128, 512) / 23).bfloat16().cuda()
        w_uv = (torch.randn(H, 512, 128) / 23).bfloat16().cuda()
        out = torch.empty(B, H, 128, dtype=torch.bfloat16, device="cuda")
        ws = mla.alloc_workspace(cache, H, torch.bfloat16)
        mla.mla_append_absorb(cache, h.cuda(), wd.cuda(), wk.cuda(), tseq, tpos, 10000.0,
                              seq_len, q_nope, q_pe, w_uk, w_uv, 1.0 / math.sqrt(192.0), out,
                              None, ws)
    else:
        mla.mla_append(cache, h.cuda(), wd.cuda(), wk.cuda(), tseq, tpos, 10000.0)
    torch.cuda.synchronize()
    exact = omla.append_rows_exact(h.double().numpy(), wd.double().numpy(), wk.double().numpy(),
                                   np.array(positions, dtype=np.float64), 10000.0)
    stored, _, _ = omla.quantize_rows(exact, "bf16")
    idx = [int(starts[s]) + p for s, p in zip(seq, positions)]
    got = cache.rows[torch.tensor(idx, device="cuda")].cpu().double().numpy()
    bound = _dot_bound(h.double().numpy(), wd.double().numpy(), wk.double().numpy(), positions,
                       10000.0)
    tie = _near_tie_bf16(exact, bound)
    mism = (got != stored) & ~tie
    log(f"  fused={fused}: {int((got != stored).sum())} of {got.size} differ, "
        f"{int(tie.sum())} near ties, {int(mism.sum())} off-tie mismatches")
    assert not mism.any()
    changed = torch.nonzero(torch.any(before.view(torch.int16) != cache.rows.view(torch.int16),
                                      dim=1)).flatten().cpu().tolist()
    assert set(changed) <= set(idx)


# ---------------------------------------------------------------- YaRN
YARN = dict(base=10000.0, scale=40.0, alpha=1.0, beta=32.0, orig_context=4096)


def _append_yarn(cache, h, wd, wk, seq, pos):
    mla = _mla()
    mla.mla_append_yarn(cache, h.cuda(), wd.cuda(), wk.cuda(),
                        torch.tensor(seq, dtype=torch.int32).cuda(),
                        torch.tensor(pos, dtype=torch.int32).cuda(), **YARN)
    torch.cuda.synchronize()


def _yarn_freq():
    return omla.yarn_inv_freq(YARN["base"], YARN["scale"], YARN["alpha"], YARN["beta"],
                              YARN["orig_context"])


def test_yarn_rope_indexing_exact_unit_probe():
    """With unit inputs pair i of the stored key is at angle pos * theta'_i
    (the YaRN frequency: kept, slowed 40x, or mixed), within 1e-6 rad of the
    fp64 value, at positions up to 131071, in an fp32 cache."""
    dm = 64
    positions = [0, 1, 3, 4095, 4096, 40000, 100000, 131071]
    n = len(positions)
    cache, starts = _cache("f32", [131072, 9])
    before = cache.rows.clone()
    h = torch.zeros(n, dm)
    h[:, 0] = 1.0
    wd = torch.zeros(512, dm)
    wd[3, 0] = 1.0
    wk = torch.zeros(64, dm)
    wk[0::2, 0] = 1.0
    _append_yarn(cache, h, wd, wk, [0] * n, positions)
    rows = cache.rows.cpu().double().numpy()
    inv = _yarn_freq()
    plain = omla.rope_inv_freq(YARN["base"])
    assert np.any(inv != plain)                    # the probe does see a different table
    worst = 0.0
    for p in positions:
        r = rows[int(starts[0]) + p]
        assert r[3] == 1.0 and np.count_nonzero(r[:512]) == 1
        for i in range(32):
            ang = math.atan2(r[512 + 2 * i + 1], r[512 + 2 * i])
            want = math.remainder(p * float(inv[i]), 2 * math.pi)
            d = abs(math.remainder(ang - want, 2 * math.pi))
            worst = max(worst, d)
            assert d < 1e-6, (p, i, ang, want)
    log(f"  YaRN: worst RoPE angle error {worst:.2e} rad")
    changed = np.nonzero(np.any(_bits(before) != _bits(cache.rows), axis=1))[0]
    assert sorted(changed.tolist()) == sorted(int(starts[0]) + p for p in positions)


@pytest.mark.parametrize("n_tok", [7, 64])
def test_append_yarn_bf16_values(n_tok):
    """bf16 rows written with YaRN frequencies equal the oracle's rounding of
    the exact rows (off the rounding midpoints), at positions up to 131071."""
    rng = np.random.default_rng(50 + n_tok)
    dm = 2048
    caps = [131072, 257]
    cache, starts = _cache("bf16", caps)
    before = cache.rows.clone()
    h = torch.from_numpy(rng.standard_normal((n_tok, dm)).astype(np.float32)).bfloat16()
    wd = torch.from_numpy((rng.standard_normal((512, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    wk = torch.from_numpy((rng.standard_normal((64, dm)) / math.sqrt(dm)).astype(np.float32)).bfloat16()
    seq = [i % 2 for i in range(n_tok)]
    # distinct slots per sequence, the last slot of each among them
    picks = {s: list(rng.choice(caps[s] - 1, size=seq.count(s) - 1, replace=False)) + [caps[s] - 1]
             for s in (0, 1)}
    pos = [int(picks[s].pop()) for s in seq]
    _append_yarn(cache, h, wd, wk, seq, pos)
    exact = omla.append_rows_exact(h.double().numpy(), wd.double().numpy(), wk.double().numpy(),
                                   np.array(pos, dtype=np.float64), YARN["base"], _yarn_freq())
    stored, _, _ = omla.quantize_rows(exact, "bf16")
    rows = cache.rows.cpu().double().numpy()
    got = np.stack([rows[int(starts[s]) + p] for s, p in zip(seq, pos)])
    bound = _dot_bound(h.double().numpy(), wd.double().numpy(), wk.double().numpy(), pos,
                       YARN["base"])
    tie = _near_tie_bf16(exact, bound)
    mism = (got != stored) & ~tie
    log(f"  YaRN bf16 n_tok={n_tok}: {int((got != stored).sum())} of {got.size} differ, "
        f"{int(tie.sum())} near ties, {int(mism.sum())} off-tie mismatches")
    assert not mism.any()
    assert np.all(np.abs(got - exact) <= np.ldexp(1.0, np.frexp(exact)[1] - 8) + bound)
    changed = np.nonzero(np.any(_bits(before) != _bits(cache.rows), axis=1))[0]
    assert set(changed.tolist()) <= {int(starts[s]) + p for s, p in zip(seq, pos)}
