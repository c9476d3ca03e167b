"""The C-ABI library on the host: it loads, exports every declared entry
point, and rejects invalid arguments before any HIP call (so these run
without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmla.h")

mla = pytest.importorskip("head_latent_attention_14_amd")
lib = mla.lib

FAKE = 0x100000      # a non-null address; never dereferenced on the error paths tested


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mla_status_t|const char\*|int|float)\s+(mla_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == {"mla_append", "mla_decode_workspace_size", "mla_decode",
                          "mla_decode_absorb", "mla_decode_attend", "mla_decode_combine",
                          "mla_decode_attend_combine",
                          "mla_append_absorb", "mla_decode_noalloc", "mla_append_yarn",
                          "mla_yarn_softmax_factor", "mla_append_paged", "mla_decode_paged",
                          "mla_append_yarn_paged",
                          "mla_prefill_workspace_size", "mla_prefill", "mla_prefill_paged",
                          "mla_status_string", "mla_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
        assert getattr(lib, n) is not None
    assert sorted(mla.EXPORTED) == names


def test_abi_version_and_constants_match_header():
    src = open(HEADER).read()
    ver = int(re.search(r"#define MLA_ABI_VERSION (\d+)", src).group(1))
    assert mla.mla_abi_version() == ver
    for name, val in [("MLA_D_C", 512), ("MLA_D_R", 64), ("MLA_D_ROW", 576)]:
        assert int(re.search(rf"#define {name} (\d+)", src).group(1)) == val
    for name in ["MLA_OK", "MLA_ERR_INVALID_ARGUMENT", "MLA_ERR_UNSUPPORTED",
                 "MLA_ERR_WORKSPACE_TOO_SMALL", "MLA_ERR_HIP"]:
        assert int(re.search(rf"{name} = (\d+)", src).group(1)) == getattr(mla, name)
    for name in ["MLA_DTYPE_F32", "MLA_DTYPE_BF16", "MLA_DTYPE_FP8_E4M3"]:
        assert int(re.search(rf"{name} = (\d+)", src).group(1)) == getattr(mla, name)


def test_status_strings():
    assert mla.mla_status_string(0) == "ok"
    assert "workspace" in mla.mla_status_string(3)
    assert mla.mla_status_string(99) == "unknown status"


def _cache(dtype=mla.MLA_DTYPE_BF16, d_c=512, d_r=64, B=4, rows=100, scale=None):
    return mla.mla_cache_t(dtype, d_c, d_r, B, rows, FAKE, scale, FAKE, FAKE)


def _decode(cache, act=mla.MLA_DTYPE_BF16, H=16, scale=0.07, ws=FAKE, ws_bytes=1 << 40,
            null=None):
    args = dict(seq_len=FAKE, q_nope=FAKE, q_pe=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE)
    if null:
        args[null] = None
    c = ctypes.byref(cache) if cache is not None else None
    return lib.mla_decode(c, args["seq_len"], args["q_nope"], args["q_pe"], args["w_uk"],
                          args["w_uv"], act, H, scale, args["out"], None, ws, ws_bytes, None)


@pytest.mark.parametrize("null", ["seq_len", "q_nope", "q_pe", "w_uk", "w_uv", "out"])
def test_decode_null_pointers(null):
    assert _decode(_cache(), null=null) == mla.MLA_ERR_INVALID_ARGUMENT


def test_decode_validation():
    E = mla
    assert _decode(None) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(d_c=256)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(d_r=32)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(B=0)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(rows=0)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(dtype=7)) == E.MLA_ERR_INVALID_ARGUMENT
    # fp8 cache needs its scales
    assert _decode(_cache(dtype=E.MLA_DTYPE_FP8_E4M3)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(), H=0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(), H=24) == E.MLA_ERR_UNSUPPORTED
    assert _decode(_cache(), scale=0.0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(), scale=float("nan")) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(), ws=None) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(), ws=FAKE + 64) == E.MLA_ERR_INVALID_ARGUMENT     # not 256-aligned
    # unsupported dtype pairs
    assert _decode(_cache(), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    assert _decode(_cache(dtype=E.MLA_DTYPE_F32), act=E.MLA_DTYPE_BF16) == E.MLA_ERR_UNSUPPORTED
    assert _decode(_cache(dtype=E.MLA_DTYPE_FP8_E4M3, scale=FAKE),
                   act=E.MLA_DTYPE_FP8_E4M3) == E.MLA_ERR_UNSUPPORTED
    # too small a workspace
    need = mla.mla_decode_workspace_size(4, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    assert _decode(_cache(), ws_bytes=need - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    # the stage entry points validate the same way
    for name in mla.DECODE_STAGES:
        fn = getattr(lib, name)
        assert fn(None, FAKE, FAKE, FAKE, FAKE, FAKE, E.MLA_DTYPE_BF16, 16, 0.07, FAKE, None,
                  FAKE, 1 << 40, None) == E.MLA_ERR_INVALID_ARGUMENT
        c = _cache()
        assert fn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, E.MLA_DTYPE_BF16, 24, 0.07,
                  FAKE, None, FAKE, 1 << 40, None) == E.MLA_ERR_UNSUPPORTED
        assert fn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, E.MLA_DTYPE_BF16, 16, 0.07,
                  FAKE, None, FAKE, need - 1, None) == E.MLA_ERR_WORKSPACE_TOO_SMALL


def test_workspace_size_query():
    E = mla
    n16 = mla.mla_decode_workspace_size(64, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    n128 = mla.mla_decode_workspace_size(64, 128, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    assert 0 < n16 < n128 and n16 % 256 == 0
    # does not depend on lengths, grows with the number of sequences
    assert mla.mla_decode_workspace_size(65, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16) >= n16
    with pytest.raises(mla.MlaError):
        mla.mla_decode_workspace_size(0, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    with pytest.raises(mla.MlaError):
        mla.mla_decode_workspace_size(4, 8, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    assert lib.mla_decode_workspace_size(4, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16, None) == \
        E.MLA_ERR_INVALID_ARGUMENT


def _append(cache, n_tok=4, d_model=128, act=mla.MLA_DTYPE_BF16, base=10000.0, null=None):
    args = dict(h=FAKE, w_dkv=FAKE, w_kr=FAKE, tok_seq=FAKE, tok_pos=FAKE)
    if null:
        args[null] = None
    c = ctypes.byref(cache) if cache is not None else None
    return lib.mla_append(c, args["h"], n_tok, d_model, args["w_dkv"], args["w_kr"], act,
                          args["tok_seq"], args["tok_pos"], base, None)


def test_append_validation():
    E = mla
    assert _append(None) == E.MLA_ERR_INVALID_ARGUMENT
    for null in ["h", "w_dkv", "w_kr", "tok_seq", "tok_pos"]:
        assert _append(_cache(), null=null) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), n_tok=-1) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), d_model=100) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), d_model=0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), base=0.0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), base=float("inf")) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append(_cache(), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    assert _append(_cache(dtype=E.MLA_DTYPE_FP8_E4M3)) == E.MLA_ERR_INVALID_ARGUMENT
    # zero tokens: a no-op that launches nothing
    assert _append(_cache(), n_tok=0) == E.MLA_OK


def _append_absorb(cache, n_tok=4, d_model=128, act=mla.MLA_DTYPE_BF16, base=10000.0, H=16,
                   scale=0.07, ws=FAKE, ws_bytes=1 << 40, null=None):
    args = dict(h=FAKE, w_dkv=FAKE, w_kr=FAKE, tok_seq=FAKE, tok_pos=FAKE, seq_len=FAKE,
                q_nope=FAKE, q_pe=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE)
    if null:
        args[null] = None
    c = ctypes.byref(cache) if cache is not None else None
    return lib.mla_append_absorb(c, args["h"], n_tok, d_model, args["w_dkv"], args["w_kr"],
                                 args["tok_seq"], args["tok_pos"], base, args["seq_len"],
                                 args["q_nope"], args["q_pe"], args["w_uk"], args["w_uv"], act,
                                 H, scale, args["out"], None, ws, ws_bytes, None)


def test_append_absorb_validation():
    # both argument sets are checked before anything is launched
    E = mla
    assert _append_absorb(None) == E.MLA_ERR_INVALID_ARGUMENT
    for null in ["h", "w_dkv", "w_kr", "tok_seq", "tok_pos", "seq_len", "q_nope", "q_pe",
                 "w_uk", "w_uv", "out"]:
        assert _append_absorb(_cache(), null=null) == E.MLA_ERR_INVALID_ARGUMENT, null
    assert _append_absorb(_cache(), d_model=100) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append_absorb(_cache(), base=0.0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append_absorb(_cache(), scale=0.0) == E.MLA_ERR_INVALID_ARGUMENT
    assert _append_absorb(_cache(), H=24) == E.MLA_ERR_UNSUPPORTED
    assert _append_absorb(_cache(), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    assert _append_absorb(_cache(), ws=FAKE + 64) == E.MLA_ERR_INVALID_ARGUMENT
    need = mla.mla_decode_workspace_size(4, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    assert _append_absorb(_cache(), ws_bytes=need - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL


# ---------------------------------------------------------------- binding checks
# The binding checks every tensor against the cache's B, q_nope's H, the
# activation dtype and the cache's device before any foreign call; these run
# on CPU tensors (the checks fire before the "device tensors" check).
import torch  # noqa: E402


def _binding_problem(B=3, H=16, act=torch.bfloat16, cache_dt=torch.bfloat16, n_tok=2, dm=64):
    rows = torch.zeros(50, 576, dtype=cache_dt)
    cache = mla.LatentCache(rows=rows, seq_start=torch.arange(B, dtype=torch.int64) * 10,
                            seq_capacity=torch.full((B,), 10, dtype=torch.int32),
                            row_scale=torch.ones(50) if cache_dt == torch.uint8 else None)
    d = dict(seq_len=torch.ones(B, dtype=torch.int32), q_nope=torch.zeros(B, H, 128, dtype=act),
             q_pe=torch.zeros(B, H, 64, dtype=act), w_uk=torch.zeros(H, 128, 512, dtype=act),
             w_uv=torch.zeros(H, 512, 128, dtype=act), out=torch.zeros(B, H, 128, dtype=act),
             lse=torch.zeros(B, H), workspace=torch.zeros(256, dtype=torch.uint8))
    a = dict(h=torch.zeros(n_tok, dm, dtype=act), w_dkv=torch.zeros(512, dm, dtype=act),
             w_kr=torch.zeros(64, dm, dtype=act), tok_seq=torch.zeros(n_tok, dtype=torch.int32),
             tok_pos=torch.zeros(n_tok, dtype=torch.int32))
    return cache, d, a


def test_binding_accepts_consistent_shapes_then_wants_device_tensors():
    cache, d, a = _binding_problem()
    assert mla.check_decode_args(cache, **d) == 16
    mla.check_append_args(cache, **a)
    with pytest.raises(ValueError, match="device tensors"):
        mla.mla_decode(cache, softmax_scale=0.07, **d)


@pytest.mark.parametrize("name,bad", [
    ("q_nope", torch.zeros(2, 16, 128, dtype=torch.bfloat16)),     # fewer rows than num_seqs
    ("q_pe", torch.zeros(3, 16, 32, dtype=torch.bfloat16)),
    ("w_uk", torch.zeros(8, 128, 512, dtype=torch.bfloat16)),      # fewer heads than q_nope
    ("w_uv", torch.zeros(16, 128, 512, dtype=torch.bfloat16)),     # transposed
    ("out", torch.zeros(3, 16, 64, dtype=torch.bfloat16)),
    ("lse", torch.zeros(3, 8)),
    ("seq_len", torch.ones(4, dtype=torch.int32)),
])
def test_binding_rejects_shape_mismatch(name, bad):
    cache, d, _ = _binding_problem()
    d[name] = bad
    with pytest.raises(ValueError, match=name):
        mla.mla_decode(cache, softmax_scale=0.07, **d)
    with pytest.raises(ValueError, match=name):
        mla.PreparedDecode(cache, softmax_scale=0.07, **d)


@pytest.mark.parametrize("name,bad", [
    ("out", torch.zeros(3, 16, 128, dtype=torch.float32)),         # f32 out, bf16 activations
    ("w_uk", torch.zeros(16, 128, 512, dtype=torch.float32)),
    ("lse", torch.zeros(3, 16, dtype=torch.bfloat16)),
    ("seq_len", torch.ones(3, dtype=torch.int64)),
])
def test_binding_rejects_dtype_mismatch(name, bad):
    cache, d, _ = _binding_problem()
    d[name] = bad
    with pytest.raises(TypeError, match=name):
        mla.mla_decode(cache, softmax_scale=0.07, **d)


def test_binding_rejects_cache_and_append_mismatch():
    cache, d, a = _binding_problem()
    cache.seq_capacity = torch.full((2,), 10, dtype=torch.int32)
    with pytest.raises(ValueError, match="seq_capacity"):
        mla.mla_decode(cache, softmax_scale=0.07, **d)
    cache, d, a = _binding_problem(cache_dt=torch.uint8)
    cache.row_scale = torch.ones(49)
    with pytest.raises(ValueError, match="row_scale"):
        mla.mla_decode(cache, softmax_scale=0.07, **d)
    cache, d, a = _binding_problem()
    a["w_dkv"] = torch.zeros(512, 128, dtype=torch.bfloat16)     # d_model disagrees with h
    with pytest.raises(ValueError, match="w_dkv"):
        mla.mla_append(cache, rope_base=1e4, **a)
    cache, d, a = _binding_problem()
    a["tok_pos"] = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="tok_pos"):
        mla.mla_append_absorb(cache, rope_base=1e4, softmax_scale=0.07, **a, **d)
    cache, d, a = _binding_problem()
    a["h"] = a["h"].float()
    a["w_dkv"] = a["w_dkv"].float()
    a["w_kr"] = a["w_kr"].float()
    with pytest.raises(TypeError, match="activation dtype"):
        mla.mla_append_absorb(cache, rope_base=1e4, softmax_scale=0.07, **a, **d)


def test_decode_noalloc_validation():
    """mla_decode_noalloc checks its arguments like mla_decode, and a request
    beyond its array, before any HIP call."""
    E = mla
    f = lib.mla_decode_noalloc
    src = open(HEADER).read()
    assert int(re.search(r"#define MLA_NOALLOC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", src)
               .expand(r"\1")) << 20 == mla.MLA_NOALLOC_WORKSPACE_BYTES

    def call(c, H=16, act=E.MLA_DTYPE_BF16, null=None):
        args = dict(seq_len=FAKE, q_nope=FAKE, q_pe=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE)
        if null:
            args[null] = None
        return f(ctypes.byref(c) if c is not None else None, args["seq_len"], args["q_nope"],
                 args["q_pe"], args["w_uk"], args["w_uv"], act, H, 0.07, args["out"], None, None)

    assert call(None) == E.MLA_ERR_INVALID_ARGUMENT
    for null in ["seq_len", "q_nope", "q_pe", "w_uk", "w_uv", "out"]:
        assert call(_cache(), null=null) == E.MLA_ERR_INVALID_ARGUMENT
    assert call(_cache(d_c=256)) == E.MLA_ERR_INVALID_ARGUMENT
    assert call(_cache(), H=24) == E.MLA_ERR_UNSUPPORTED
    assert call(_cache(), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    big = _cache(dtype=E.MLA_DTYPE_FP8_E4M3, B=128, scale=FAKE)
    need = mla.mla_decode_workspace_size(128, 128, E.MLA_DTYPE_FP8_E4M3, E.MLA_DTYPE_BF16)
    assert need > mla.MLA_NOALLOC_WORKSPACE_BYTES
    assert call(big, H=128) == E.MLA_ERR_WORKSPACE_TOO_SMALL


def test_append_yarn_validation_and_softmax_factor():
    E = mla
    c = _cache()

    def call(rope, n_tok=4, null=None):
        args = dict(h=FAKE, w_dkv=FAKE, w_kr=FAKE, tok_seq=FAKE, tok_pos=FAKE)
        if null:
            args[null] = None
        r = ctypes.byref(rope) if rope is not None else None
        return lib.mla_append_yarn(ctypes.byref(c), args["h"], n_tok, 128, args["w_dkv"], args["w_kr"],
                                   E.MLA_DTYPE_BF16, args["tok_seq"], args["tok_pos"], r, None)

    good = dict(base=10000.0, scale=40.0, alpha=1.0, beta=32.0, orig_context=4096)
    assert call(None) == E.MLA_ERR_INVALID_ARGUMENT
    for k, v in [("base", 0.0), ("base", float("nan")), ("scale", 0.5), ("scale", float("inf")),
                 ("alpha", -1.0), ("beta", 1.0), ("orig_context", 0)]:
        assert call(mla.mla_yarn_t(**dict(good, **{k: v}))) == E.MLA_ERR_INVALID_ARGUMENT, k
    assert call(mla.mla_yarn_t(**good), null="h") == E.MLA_ERR_INVALID_ARGUMENT
    assert call(mla.mla_yarn_t(**good), n_tok=-1) == E.MLA_ERR_INVALID_ARGUMENT
    # n_tok == 0 is a valid no-op that touches nothing
    assert call(mla.mla_yarn_t(**good), n_tok=0) == E.MLA_OK
    # the paged form checks the pool first, then the same frequency parameters
    pc = _paged()

    def call_p(rope, n_tok=4):
        r = ctypes.byref(rope) if rope is not None else None
        return lib.mla_append_yarn_paged(ctypes.byref(pc), FAKE, n_tok, 128, FAKE, FAKE,
                                         E.MLA_DTYPE_BF16, FAKE, FAKE, r, None)

    assert call_p(None) == E.MLA_ERR_INVALID_ARGUMENT
    assert call_p(mla.mla_yarn_t(**dict(good, beta=0.5))) == E.MLA_ERR_INVALID_ARGUMENT
    assert call_p(mla.mla_yarn_t(**good), n_tok=0) == E.MLA_OK
    assert lib.mla_append_yarn_paged(None, FAKE, 4, 128, FAKE, FAKE, E.MLA_DTYPE_BF16, FAKE, FAKE,
                                     ctypes.byref(mla.mla_yarn_t(**good)), None) \
        == E.MLA_ERR_INVALID_ARGUMENT
    import math
    assert mla.mla_yarn_softmax_factor(1.0) == 1.0
    assert mla.mla_yarn_softmax_factor(0.25) == 1.0
    assert mla.mla_yarn_softmax_factor(float("nan")) == 1.0
    assert abs(mla.mla_yarn_softmax_factor(math.exp(10.0)) - 4.0) < 1e-6


def _paged(dtype=mla.MLA_DTYPE_BF16, B=4, P=64, max_pages=8, total_pages=20, table=FAKE,
           scale=None, d_c=512):
    return mla.mla_paged_cache_t(dtype, d_c, 64, B, P, max_pages, total_pages, FAKE, scale, table)


def test_paged_validation():
    """Paged entry points check the pool, the page size and the table before
    any HIP call."""
    E = mla

    def dec(c, H=16, act=E.MLA_DTYPE_BF16, ws_bytes=1 << 40):
        return lib.mla_decode_paged(ctypes.byref(c) if c is not None else None, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, act, H, 0.07, FAKE, None, FAKE, ws_bytes, None)

    def app(c, n_tok=4):
        return lib.mla_append_paged(ctypes.byref(c) if c is not None else None, FAKE, n_tok, 128,
                                    FAKE, FAKE, E.MLA_DTYPE_BF16, FAKE, FAKE, 10000.0, None)

    def pf(c, H=16, ws_bytes=1 << 40):
        return lib.mla_prefill_paged(ctypes.byref(c) if c is not None else None, FAKE, FAKE, 64,
                                     1000, FAKE, FAKE, FAKE, FAKE, E.MLA_DTYPE_BF16, H, 0.07, FAKE,
                                     None, FAKE, ws_bytes, None)

    for f in (dec, app, pf):
        assert f(None) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(P=48)) == E.MLA_ERR_INVALID_ARGUMENT        # not a multiple of 32
        assert f(_paged(P=0)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(max_pages=0)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(total_pages=0)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(table=None)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(B=0)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(d_c=256)) == E.MLA_ERR_INVALID_ARGUMENT
        assert f(_paged(dtype=E.MLA_DTYPE_FP8_E4M3)) == E.MLA_ERR_INVALID_ARGUMENT  # no row_scale
        # capacities must fit int32 positions
        assert f(_paged(P=1 << 16, max_pages=1 << 16)) == E.MLA_ERR_UNSUPPORTED
    assert dec(_paged(), H=24) == E.MLA_ERR_UNSUPPORTED
    need = mla.mla_decode_workspace_size(4, 16, E.MLA_DTYPE_BF16, E.MLA_DTYPE_BF16)
    assert dec(_paged(), ws_bytes=need - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    assert app(_paged(), n_tok=0) == E.MLA_OK                      # a no-op
    # paged prefill: any head count, the prefill workspace, f32 pools unsupported
    need = mla.mla_prefill_workspace_size(4, 3, 64, 1000)
    assert pf(_paged(), H=3, ws_bytes=need - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    assert pf(_paged(dtype=E.MLA_DTYPE_F32)) == E.MLA_ERR_UNSUPPORTED


def test_paged_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    pc = mla.PagedLatentCache(rows=torch.zeros(128, 576, dtype=torch.bfloat16),
                              block_table=torch.zeros(2, 2, dtype=torch.int32), page_tokens=64)
    assert pc.num_seqs == 2 and pc.dtype == mla.MLA_DTYPE_BF16
    pc.check()
    with pytest.raises((ValueError, TypeError)):
        mla.PagedLatentCache(rows=torch.zeros(100, 576, dtype=torch.bfloat16),
                             block_table=torch.zeros(2, 2, dtype=torch.int32), page_tokens=64).check()
    with pytest.raises((ValueError, TypeError)):
        mla.PagedLatentCache(rows=torch.zeros(128, 576, dtype=torch.bfloat16),
                             block_table=torch.zeros(2, 2, dtype=torch.int64), page_tokens=64).check()
    with pytest.raises((ValueError, TypeError)):
        mla.PagedLatentCache(rows=torch.zeros(128, 576, dtype=torch.uint8),
                             block_table=torch.zeros(2, 2, dtype=torch.int32), page_tokens=64).check()


def test_prefill_validation():
    """mla_prefill checks the cache, counts, dtypes, pointers and workspace
    before any HIP call."""
    E = mla

    def pf(c, n_q=64, kv=1000, H=16, act=E.MLA_DTYPE_BF16, scale=0.07, ws=FAKE,
           ws_bytes=1 << 40, null=None):
        args = dict(seq_len=FAKE, q_start=FAKE, q_nope=FAKE, q_pe=FAKE, w_uk=FAKE, w_uv=FAKE,
                    out=FAKE)
        if null:
            args[null] = None
        return lib.mla_prefill(ctypes.byref(c) if c is not None else None, args["seq_len"],
                               args["q_start"], n_q, kv, args["q_nope"], args["q_pe"],
                               args["w_uk"], args["w_uv"], act, H, scale, args["out"], None, ws,
                               ws_bytes, None)

    assert pf(None) == E.MLA_ERR_INVALID_ARGUMENT
    for null in ["seq_len", "q_start", "q_nope", "q_pe", "w_uk", "w_uv", "out"]:
        assert pf(_cache(), null=null) == E.MLA_ERR_INVALID_ARGUMENT, null
    assert pf(_cache(), ws=None) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), ws=FAKE + 64) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), H=0) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), H=2000) == E.MLA_ERR_UNSUPPORTED
    assert pf(_cache(), n_q=-1) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), kv=-1) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), scale=0.0) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), scale=float("inf")) == E.MLA_ERR_INVALID_ARGUMENT
    # f32 caches and non-bf16 activations are not supported
    assert pf(_cache(dtype=E.MLA_DTYPE_F32)) == E.MLA_ERR_UNSUPPORTED
    assert pf(_cache(), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    # fp6 caches pass validation up to the workspace check; their scales are in the rows
    assert pf(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX), ws_bytes=1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    assert pf(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX, scale=FAKE)) == E.MLA_ERR_INVALID_ARGUMENT
    assert pf(_cache(), act=9) == E.MLA_ERR_INVALID_ARGUMENT
    # any head count; the workspace grows with heads and rows
    n1 = mla.mla_prefill_workspace_size(4, 1, 64, 1000)
    n3 = mla.mla_prefill_workspace_size(4, 3, 64, 1000)
    n3b = mla.mla_prefill_workspace_size(4, 3, 64, 5000)
    assert 0 < n1 < n3 < n3b and n1 % 256 == 0
    assert pf(_cache(), H=3, ws_bytes=n3 - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(mla.MlaError):
        mla.mla_prefill_workspace_size(0, 16, 64, 1000)
    assert lib.mla_prefill_workspace_size(4, 16, 64, 1000, None) == E.MLA_ERR_INVALID_ARGUMENT
    # sizes past what the launches index
    assert lib.mla_prefill_workspace_size(4, 16, 1 << 40, 1000, ctypes.byref(ctypes.c_size_t())) \
        == E.MLA_ERR_UNSUPPORTED


def test_prefill_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    cache = mla.LatentCache(rows=torch.zeros(64, 576, dtype=torch.bfloat16),
                            seq_start=torch.tensor([0, 32], dtype=torch.int64),
                            seq_capacity=torch.tensor([32, 32], dtype=torch.int32))
    H, n_q = 2, 5
    ok = dict(seq_len=torch.zeros(2, dtype=torch.int32), q_start=torch.zeros(3, dtype=torch.int32),
              q_nope=torch.zeros(n_q, H, 128, dtype=torch.bfloat16),
              q_pe=torch.zeros(n_q, H, 64, dtype=torch.bfloat16),
              w_uk=torch.zeros(H, 128, 512, dtype=torch.bfloat16),
              w_uv=torch.zeros(H, 512, 128, dtype=torch.bfloat16),
              out=torch.zeros(n_q, H, 128, dtype=torch.bfloat16))

    def call(**over):
        a = dict(ok, **over)
        mla.mla_prefill(cache, a["seq_len"], a["q_start"], 64, a["q_nope"], a["q_pe"], a["w_uk"],
                        a["w_uv"], 0.07, a["out"], None, torch.zeros(256, dtype=torch.uint8))

    for bad in [dict(q_start=torch.zeros(2, dtype=torch.int32)),
                dict(q_pe=torch.zeros(n_q, H, 32, dtype=torch.bfloat16)),
                dict(out=torch.zeros(n_q, H, 128, dtype=torch.float32)),
                dict(q_nope=torch.zeros(n_q, H, 128, dtype=torch.float32)),
                dict(w_uv=torch.zeros(H, 128, 512, dtype=torch.bfloat16))]:
        with pytest.raises((ValueError, TypeError)):
            call(**bad)


def test_fp6_cache_validation():
    """The fp6 cache carries its scales in the rows: row_scale must be NULL;
    it pairs with bf16 activations only; the workspace is sized as for the
    other 8/16-bit caches."""
    E = mla
    assert _decode(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX, scale=FAKE)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX), act=E.MLA_DTYPE_F32) == E.MLA_ERR_UNSUPPORTED
    need = mla.mla_decode_workspace_size(4, 16, E.MLA_DTYPE_FP6_E2M3_MX, E.MLA_DTYPE_BF16)
    assert need > 0
    assert _decode(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX), ws_bytes=need - 1) == E.MLA_ERR_WORKSPACE_TOO_SMALL
    assert _append(_cache(dtype=E.MLA_DTYPE_FP6_E2M3_MX, scale=FAKE)) == E.MLA_ERR_INVALID_ARGUMENT
    assert _decode(_cache(dtype=4)) == E.MLA_ERR_INVALID_ARGUMENT
    torch = pytest.importorskip("torch")
    c = mla.LatentCache(rows=torch.zeros(8, 464, dtype=torch.uint8),
                        seq_start=torch.tensor([0], dtype=torch.int64),
                        seq_capacity=torch.tensor([8], dtype=torch.int32))
    assert c.dtype == E.MLA_DTYPE_FP6_E2M3_MX
    c.check()
    with pytest.raises((ValueError, TypeError)):
        mla.LatentCache(rows=torch.zeros(8, 464, dtype=torch.uint8),
                        seq_start=torch.tensor([0], dtype=torch.int64),
                        seq_capacity=torch.tensor([8], dtype=torch.int32),
                        row_scale=torch.zeros(8)).check()
