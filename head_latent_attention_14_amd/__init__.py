"""Python binding of libmla (MLA decode over a compressed latent cache on MI355X).

Argument marshalling only: every step runs in the HIP kernels of libmla.so,
reached through its C ABI (include/libmla.h). PyTorch supplies device memory
and the current stream. Importing this package raises if libmla.so has not
been built (`python -m head_latent_attention_14_amd.build`); there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4

MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1
MLA_DTYPE_FP8_E4M3 = 2

D_C, D_R, D_ROW, D_NOPE, D_V = 512, 64, 576, 128, 128

EXPORTED = ["mla_append", "mla_decode_workspace_size", "mla_decode", "mla_decode_absorb",
            "mla_decode_attend", "mla_decode_combine", "mla_decode_attend_combine",
            "mla_append_absorb", "mla_status_string",
            "mla_abi_version"]
DECODE_STAGES = ["mla_decode_absorb", "mla_decode_attend", "mla_decode_combine",
                 "mla_decode_attend_combine"]


class mla_cache_t(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("d_c", ctypes.c_int32),
        ("d_r", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("total_rows", ctypes.c_int64),
        ("rows", ctypes.c_void_p),
        ("row_scale", ctypes.c_void_p),
        ("seq_start", ctypes.c_void_p),
        ("seq_capacity", ctypes.c_void_p),
    ]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"libmla.so not built at {path}; run "
                          "`python -m head_latent_attention_14_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    C = ctypes.POINTER(mla_cache_t)
    lib.mla_append.argtypes = [C, P, I32, I32, P, P, ctypes.c_int, P, P, F32, P]
    lib.mla_append.restype = ctypes.c_int
    lib.mla_decode_workspace_size.argtypes = [I32, I32, ctypes.c_int, ctypes.c_int,
                                              ctypes.POINTER(SZ)]
    lib.mla_decode_workspace_size.restype = ctypes.c_int
    for name in ["mla_decode", "mla_decode_absorb", "mla_decode_attend", "mla_decode_combine",
                 "mla_decode_attend_combine"]:
        fn = getattr(lib, name)
        fn.argtypes = [C, P, P, P, P, P, ctypes.c_int, I32, F32, P, P, P, SZ, P]
        fn.restype = ctypes.c_int
    lib.mla_append_absorb.argtypes = [C, P, I32, I32, P, P, P, P, F32,
                                      P, P, P, P, P, ctypes.c_int, I32, F32, P, P, P, SZ, P]
    lib.mla_append_absorb.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = ctypes.c_int
    return lib


lib = _load()


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.mla_status_string(status).decode()} (status {status})")


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MlaError(status, where)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MLA_DTYPE_F32
    if t == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return MLA_DTYPE_FP8_E4M3
    raise TypeError(f"no libmla dtype for {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmla takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmla takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclasses.dataclass
class LatentCache:
    """Device tensors of a ragged latent cache (see mla_cache_t)."""
    rows: torch.Tensor                 # [total_rows, 576] f32 | bf16 | uint8 codes
    seq_start: torch.Tensor            # [B] int64
    seq_capacity: torch.Tensor         # [B] int32
    row_scale: Optional[torch.Tensor] = None   # [total_rows] f32 (fp8 only)

    @property
    def dtype(self) -> int:
        return dtype_code(self.rows.dtype)

    @property
    def num_seqs(self) -> int:
        return self.seq_start.shape[0]

    def struct(self) -> mla_cache_t:
        if self.seq_start.dtype != torch.int64 or self.seq_capacity.dtype != torch.int32:
            raise TypeError("seq_start must be int64 and seq_capacity int32")
        if self.rows.dim() != 2 or self.rows.shape[1] != D_ROW:
            raise ValueError("rows must be [total_rows, 576]")
        return mla_cache_t(self.dtype, D_C, D_R, self.num_seqs, self.rows.shape[0],
                           _ptr(self.rows), _ptr(self.row_scale), _ptr(self.seq_start),
                           _ptr(self.seq_capacity))


def mla_abi_version() -> int:
    return lib.mla_abi_version()


def mla_status_string(status: int) -> str:
    return lib.mla_status_string(status).decode()


def mla_append(cache: LatentCache, h: torch.Tensor, w_dkv: torch.Tensor, w_kr: torch.Tensor,
               tok_seq: torch.Tensor, tok_pos: torch.Tensor, rope_base: float,
               stream=None) -> None:
    """Write (W_DKV h) || RoPE(W_KR h, pos) into the cache (see libmla.h)."""
    if tok_seq.dtype != torch.int32 or tok_pos.dtype != torch.int32:
        raise TypeError("tok_seq and tok_pos must be int32")
    n_tok, d_model = h.shape
    st = ctypes.byref(cache.struct())
    _check(lib.mla_append(st, _ptr(h), n_tok, d_model, _ptr(w_dkv), _ptr(w_kr),
                          dtype_code(h.dtype), _ptr(tok_seq), _ptr(tok_pos),
                          float(rope_base), _stream(stream)), "mla_append")


def mla_append_absorb(cache: LatentCache, h: torch.Tensor, w_dkv: torch.Tensor,
                      w_kr: torch.Tensor, tok_seq: torch.Tensor, tok_pos: torch.Tensor,
                      rope_base: float, seq_len: torch.Tensor, q_nope: torch.Tensor,
                      q_pe: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                      softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                      workspace: torch.Tensor, stream=None) -> None:
    """mla_append then mla_decode_absorb, in one launch where it applies (see libmla.h)."""
    if tok_seq.dtype != torch.int32 or tok_pos.dtype != torch.int32 or seq_len.dtype != torch.int32:
        raise TypeError("tok_seq, tok_pos and seq_len must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    n_tok, d_model = h.shape
    B, H, _ = q_nope.shape
    st = ctypes.byref(cache.struct())
    _check(lib.mla_append_absorb(st, _ptr(h), n_tok, d_model, _ptr(w_dkv), _ptr(w_kr),
                                 _ptr(tok_seq), _ptr(tok_pos), float(rope_base), _ptr(seq_len),
                                 _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                                 dtype_code(q_nope.dtype), H, float(softmax_scale), _ptr(out),
                                 _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_append_absorb")


def mla_decode_workspace_size(num_seqs: int, n_heads: int, cache_dtype: int,
                              act_dtype: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.mla_decode_workspace_size(num_seqs, n_heads, cache_dtype, act_dtype,
                                         ctypes.byref(n)), "mla_decode_workspace_size")
    return n.value


def alloc_workspace(cache: LatentCache, n_heads: int, act_dtype: torch.dtype,
                    device=None) -> torch.Tensor:
    n = mla_decode_workspace_size(cache.num_seqs, n_heads, cache.dtype, dtype_code(act_dtype))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or cache.rows.device)


def _decode_call(name, cache, seq_len, q_nope, q_pe, w_uk, w_uv, softmax_scale, out, lse,
                 workspace, stream=None):
    if seq_len.dtype != torch.int32:
        raise TypeError("seq_len must be int32")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    B, H, _ = q_nope.shape
    st = ctypes.byref(cache.struct())
    _check(getattr(lib, name)(st, _ptr(seq_len), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk),
                              _ptr(w_uv), dtype_code(q_nope.dtype), H, float(softmax_scale),
                              _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                              _stream(stream)), name)


def mla_decode(cache: LatentCache, seq_len: torch.Tensor, q_nope: torch.Tensor,
               q_pe: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
               softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
               workspace: torch.Tensor, stream=None) -> None:
    """o[B,H,128] (and lse[B,H]) of MLA decode over the latent cache (see libmla.h)."""
    _decode_call("mla_decode", cache, seq_len, q_nope, q_pe, w_uk, w_uv, softmax_scale, out,
                 lse, workspace, stream)


def mla_decode_absorb(*args, **kw) -> None:
    """Stage 1 of mla_decode (same arguments)."""
    _decode_call("mla_decode_absorb", *args, **kw)


def mla_decode_attend(*args, **kw) -> None:
    """Stage 2 of mla_decode (same arguments)."""
    _decode_call("mla_decode_attend", *args, **kw)


def mla_decode_combine(*args, **kw) -> None:
    """Stage 3 of mla_decode (same arguments)."""
    _decode_call("mla_decode_combine", *args, **kw)


def mla_decode_attend_combine(*args, **kw) -> None:
    """Stages 2 and 3 of mla_decode in one call (same arguments)."""
    _decode_call("mla_decode_attend_combine", *args, **kw)


class PreparedDecode:
    """mla_decode and its three stages with the arguments marshalled once.

    For callers that run the same decode over the same tensors many times
    (a serving loop over fixed buffers, a benchmark): the per-call cost is one
    foreign call with precomputed pointers. The tensors are kept alive by this
    object; changing their contents between calls is fine, reallocating them
    is not."""

    def __init__(self, cache: LatentCache, seq_len: torch.Tensor, q_nope: torch.Tensor,
                 q_pe: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                 softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                 workspace: torch.Tensor, stream=None):
        if seq_len.dtype != torch.int32:
            raise TypeError("seq_len must be int32")
        if lse is not None and lse.dtype != torch.float32:
            raise TypeError("lse must be float32")
        B, H, _ = q_nope.shape
        self._keep = (cache, seq_len, q_nope, q_pe, w_uk, w_uv, out, lse, workspace)
        self._st = cache.struct()
        self._args = (ctypes.byref(self._st), _ptr(seq_len), _ptr(q_nope), _ptr(q_pe),
                      _ptr(w_uk), _ptr(w_uv), dtype_code(q_nope.dtype), H,
                      float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                      workspace.numel(), _stream(stream))

    def __call__(self) -> None:
        _check(lib.mla_decode(*self._args), "mla_decode")

    def absorb(self) -> None:
        _check(lib.mla_decode_absorb(*self._args), "mla_decode_absorb")

    def attend(self) -> None:
        _check(lib.mla_decode_attend(*self._args), "mla_decode_attend")

    def combine(self) -> None:
        _check(lib.mla_decode_combine(*self._args), "mla_decode_combine")

    def attend_combine(self) -> None:
        _check(lib.mla_decode_attend_combine(*self._args), "mla_decode_attend_combine")


class PreparedAppend:
    """mla_append with the arguments marshalled once (see PreparedDecode)."""

    def __init__(self, cache: LatentCache, h: torch.Tensor, w_dkv: torch.Tensor,
                 w_kr: torch.Tensor, tok_seq: torch.Tensor, tok_pos: torch.Tensor,
                 rope_base: float, stream=None):
        if tok_seq.dtype != torch.int32 or tok_pos.dtype != torch.int32:
            raise TypeError("tok_seq and tok_pos must be int32")
        n_tok, d_model = h.shape
        self._keep = (cache, h, w_dkv, w_kr, tok_seq, tok_pos)
        self._st = cache.struct()
        self._args = (ctypes.byref(self._st), _ptr(h), n_tok, d_model, _ptr(w_dkv), _ptr(w_kr),
                      dtype_code(h.dtype), _ptr(tok_seq), _ptr(tok_pos), float(rope_base),
                      _stream(stream))

    def __call__(self) -> None:
        _check(lib.mla_append(*self._args), "mla_append")


class PreparedAppendAbsorb:
    """mla_append_absorb with the arguments marshalled once (see PreparedDecode);
    follow it with PreparedDecode.attend() and .combine() on the same decode
    arguments to complete the step."""

    def __init__(self, cache: LatentCache, h: torch.Tensor, w_dkv: torch.Tensor,
                 w_kr: torch.Tensor, tok_seq: torch.Tensor, tok_pos: torch.Tensor,
                 rope_base: float, seq_len: torch.Tensor, q_nope: torch.Tensor,
                 q_pe: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                 softmax_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                 workspace: torch.Tensor, stream=None):
        if (tok_seq.dtype != torch.int32 or tok_pos.dtype != torch.int32
                or seq_len.dtype != torch.int32):
            raise TypeError("tok_seq, tok_pos and seq_len must be int32")
        if lse is not None and lse.dtype != torch.float32:
            raise TypeError("lse must be float32")
        n_tok, d_model = h.shape
        B, H, _ = q_nope.shape
        self._keep = (cache, h, w_dkv, w_kr, tok_seq, tok_pos, seq_len, q_nope, q_pe, w_uk, w_uv,
                      out, lse, workspace)
        self._st = cache.struct()
        self._args = (ctypes.byref(self._st), _ptr(h), n_tok, d_model, _ptr(w_dkv), _ptr(w_kr),
                      _ptr(tok_seq), _ptr(tok_pos), float(rope_base), _ptr(seq_len),
                      _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
                      dtype_code(q_nope.dtype), H, float(softmax_scale), _ptr(out), _ptr(lse),
                      _ptr(workspace), workspace.numel(), _stream(stream))

    def __call__(self) -> None:
        _check(lib.mla_append_absorb(*self._args), "mla_append_absorb")
