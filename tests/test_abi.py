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
    return sorted(set(re.findall(r"^\s*(?:mla_status_t|const char\*|int)\s+(mla_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == {"mla_append", "mla_decode_workspace_size", "mla_decode",
                          "mla_decode_absorb", "mla_decode_attend", "mla_decode_combine",
                          "mla_decode_attend_combine",
                          "mla_append_absorb", "mla_status_string", "mla_abi_version"}
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
