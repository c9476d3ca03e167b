"""Paged latent cache on the GPU, through the C ABI: decode over a paged
cache equals decode over the same rows laid out contiguously, bit for bit
(and both meet the oracle's bound), for every attention kernel and several
page sizes with shuffled pages; append into a paged cache writes exactly the
rows the contiguous append writes, at the block table's rows, and skips
tokens whose block has no valid page."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.problem import OracleView
from tests.gpu_util import TOL, DeviceProblem, log, rel_l2

pytestmark = pytest.mark.gpu


def _mla():
    import head_latent_attention_14_amd as mla
    return mla


def _page(dp, P, seed):
    """A paged copy of DeviceProblem dp's cache: every sequence's capacity in
    shuffled P-row pages of a pool with spare pages, unused rows random."""
    mla = _mla()
    p = dp.p
    caps = p.seq_capacity.astype(np.int64)
    npg = (caps + P - 1) // P
    total = int(npg.sum()) + 3
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total)
    table = np.zeros((len(caps), int(npg.max())), dtype=np.int32)
    src, dst = [], []
    k = 0
    for b, c in enumerate(caps):
        table[b, :npg[b]] = perm[k:k + npg[b]]
        k += npg[b]
        t = np.arange(c)
        src.append(int(p.seq_start[b]) + t)
        dst.append(table[b, t // P].astype(np.int64) * P + t % P)
    src, dst = np.concatenate(src), np.concatenate(dst)
    rows = dp.cache.rows
    pool = torch.empty((total * P, rows.shape[1]), dtype=rows.dtype, device=rows.device)
    if rows.dtype == torch.uint8:
        pool.random_(0, 0x7E)
    else:
        pool.normal_()
    pool[torch.from_numpy(dst).cuda()] = rows[torch.from_numpy(src).cuda()]
    scale = None
    if dp.cache.row_scale is not None:
        scale = torch.rand(total * P, device=rows.device) + 0.5
        scale[torch.from_numpy(dst).cuda()] = dp.cache.row_scale[torch.from_numpy(src).cuda()]
    return mla.PagedLatentCache(rows=pool, block_table=torch.from_numpy(table).cuda(),
                                page_tokens=P, row_scale=scale)


def _decode_paged(dp, pc):
    mla = _mla()
    out = torch.full_like(dp.out, float("nan"))
    lse = torch.full_like(dp.lse, float("nan"))
    ws = mla.alloc_workspace(pc, dp.H, dp.q_nope.dtype)
    mla.mla_decode_paged(pc, dp.seq_len, dp.q_nope, dp.q_pe, dp.w_uk, dp.w_uv,
                         1.0 / math.sqrt(192.0), out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _same_bits(a, b):
    ints = {torch.float32: torch.int32, torch.bfloat16: torch.int16}
    return torch.equal(a.view(ints[a.dtype]), b.view(ints[b.dtype]))


CASES = [
    ("v2lite_bf16", [1, 33, 300, 64, 129], 32),     # streaming kernel (16 heads)
    ("v2lite_bf16", [1, 33, 300, 64, 129], 96),
    ("v2_bf16", [1, 33, 200, 97], 64),               # pair kernel (128 heads)
    ("fp8_cache", [1, 33, 200, 97], 32),             # fp8 pair kernel
    ("fp6_cache", [1, 33, 200, 97], 32),             # fp6 pair kernel (tiles widened in LDS)
    ("tiny_fp32", [256, 40], 64),                    # f32 kernel (16-token tiles)
]


@pytest.mark.parametrize("name,lengths,P", CASES)
def test_paged_decode_equals_contiguous(name, lengths, P):
    wl = W.WORKLOADS[name]
    p = W.make_problem(wl, B=len(lengths), lengths=np.array(lengths))
    dp = DeviceProblem(p)
    o_c, l_c = dp.step(poison=True)                  # contiguous (append applied if any)
    pc = _page(dp, P, seed=P + len(lengths))
    out, lse = _decode_paged(dp, pc)
    log(f"[paged] {name} lengths={lengths} P={P}")
    assert _same_bits(out, dp.out) and _same_bits(lse, dp.lse)
    ro, _ = OracleView(p).decode()
    assert rel_l2(out.double().cpu().numpy(), ro) <= TOL[wl.cache]


def test_paged_decode_full_size_v2():
    """The benchmark's 128-head shape with 64-token pages: bit for bit."""
    wl = W.WORKLOADS["v2_bf16"]
    p = W.make_problem(wl)
    dp = DeviceProblem(p)
    dp.step(poison=True)
    pc = _page(dp, 64, seed=11)
    out, lse = _decode_paged(dp, pc)
    assert _same_bits(out, dp.out) and _same_bits(lse, dp.lse)


@pytest.mark.parametrize("dtype,yarn", [("bf16", False), ("fp8", False), ("bf16", True)])
def test_paged_append_matches_contiguous_rows(dtype, yarn):
    mla = _mla()
    rng = np.random.default_rng(5)
    dm, n_tok, P = 256, 24, 64
    caps = [200, 64, 130]
    B = len(caps)
    npg = [(c + P - 1) // P for c in caps]
    total = sum(npg) + 2
    perm = rng.permutation(total)
    table = np.full((B, max(npg) + 1), -1, dtype=np.int32)   # one column past every capacity
    k = 0
    for b in range(B):
        table[b, :npg[b]] = perm[k:k + npg[b]]
        k += npg[b]
    tdt = W.TORCH_DTYPE[dtype]
    if dtype == "fp8":
        pool = torch.randint(0, 0x7E, (total * P, 576), dtype=torch.uint8).cuda()
        scale = (torch.rand(total * P) + 0.5).cuda()
        cont = torch.zeros((sum(caps), 576), dtype=torch.uint8).cuda()
        cscale = torch.ones(sum(caps)).cuda()
    else:
        pool = torch.randn(total * P, 576).to(tdt).cuda()
        scale, cont, cscale = None, torch.zeros((sum(caps), 576), dtype=tdt).cuda(), None
    starts = np.concatenate([[0], np.cumsum(caps)[:-1]])
    pc = mla.PagedLatentCache(rows=pool, block_table=torch.from_numpy(table).cuda(), page_tokens=P,
                              row_scale=scale)
    cc = mla.LatentCache(rows=cont, seq_start=torch.from_numpy(starts).cuda(),
                         seq_capacity=torch.tensor(caps, dtype=torch.int32).cuda(), row_scale=cscale)
    h = torch.randn(n_tok, dm).bfloat16().cuda()
    wd = (torch.randn(512, dm) / 16).bfloat16().cuda()
    wk = (torch.randn(64, dm) / 16).bfloat16().cuda()
    slots = rng.choice([(b, t) for b in range(B) for t in range(caps[b])], size=n_tok, replace=False)
    seq = torch.tensor([int(s[0]) for s in slots], dtype=torch.int32).cuda()
    pos = torch.tensor([int(s[1]) for s in slots], dtype=torch.int32).cuda()
    before = pool.clone()
    if yarn:                                       # YaRN frequencies (DeepSeek-V2's constants)
        mla.mla_append_yarn(pc, h, wd, wk, seq, pos)
        mla.mla_append_yarn(cc, h, wd, wk, seq, pos)
    else:
        mla.mla_append_paged(pc, h, wd, wk, seq, pos, 10000.0)
        mla.mla_append(cc, h, wd, wk, seq, pos, 10000.0)
    torch.cuda.synchronize()
    written = set()
    for (b, t) in slots:
        r = int(table[b, t // P]) * P + t % P
        c = int(starts[b]) + t
        written.add(r)
        assert torch.equal(pool[r], cont[c]), (b, t)
        if scale is not None:
            assert torch.equal(scale[r], cscale[c]), (b, t)
    changed = torch.nonzero((pool != before).any(dim=1)).flatten().tolist()
    assert set(changed) <= written
    # a position past the capacity (its block holds -1) is skipped
    snap = pool.clone()
    mla.mla_append_paged(pc, h[:1], wd, wk, torch.tensor([1], dtype=torch.int32).cuda(),
                         torch.tensor([caps[1] + 5], dtype=torch.int32).cuda(), 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(pool, snap)
