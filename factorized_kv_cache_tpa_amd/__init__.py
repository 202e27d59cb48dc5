"""Python binding of libtpa: attention over a TPA factor cache on MI355X.

Thin ctypes marshalling of the C ABI in ``include/tpa.h``; the functions
carry the same names.  Every step of the computation runs in the HIP kernels
of ``libtpa.so``; this module only turns torch tensors into device pointers
and the current HIP stream into a ``hipStream_t``.  There is no fallback: if
the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "TPAError", "Dims", "load", "library_path", "tpa_abi_version", "tpa_status_string", "tpa_supported",
    "tpa_block_tokens", "tpa_cache_bytes", "tpa_cache_append", "tpa_cache_read", "tpa_decode_workspace_bytes",
    "tpa_decode", "tpa_decode_noalloc", "TPA_DECODE_NOALLOC_MAX_BYTES", "tpa_decode_step", "tpa_decode_fq",
    "tpa_prefill_chunk", "tpa_prefill_chunk_fq", "TPA_F32", "TPA_BF16", "TPA_CACHE_NATIVE", "TPA_CACHE_E4M3",
]

TPA_F32 = 0
TPA_BF16 = 1
TPA_CACHE_NATIVE = 0
TPA_CACHE_E4M3 = 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtpa.so")
_lib = None

_EXPORTS = {
    "tpa_abi_version": ([], ctypes.c_int32),
    "tpa_status_string": ([ctypes.c_int32], ctypes.c_char_p),
    "tpa_supported": ([ctypes.c_void_p], ctypes.c_int32),
    "tpa_block_tokens": ([ctypes.c_void_p], ctypes.c_int32),
    "tpa_cache_bytes": ([ctypes.c_void_p, ctypes.c_int64], ctypes.c_int64),
    "tpa_cache_append": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int32),
    "tpa_cache_read": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
                       ctypes.c_int32),
    "tpa_decode_workspace_bytes": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32],
                                   ctypes.c_int64),
    "tpa_decode": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p], ctypes.c_int32),
    "tpa_decode_noalloc": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                            ctypes.c_int32, ctypes.c_void_p], ctypes.c_int32),
    "tpa_decode_step": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_int32,
                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p], ctypes.c_int32),
    "tpa_decode_fq": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_float, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                       ctypes.c_void_p], ctypes.c_int32),
    "tpa_prefill_chunk_fq": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int32),
    "tpa_prefill_chunk": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                           ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int32),
}


class TPAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {tpa_status_string(status)} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    """tpa_dims: h, d_h, R_K, R_V, dtype (TPA_F32 / TPA_BF16), cache_format (TPA_CACHE_NATIVE /
    TPA_CACHE_E4M3), rope_base, cache_scale[4] (E4M3 scales of A_K, B_K, A_V, B_V; 0 means 1)."""
    _fields_ = [("h", ctypes.c_int32), ("d_h", ctypes.c_int32), ("R_K", ctypes.c_int32), ("R_V", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("cache_format", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("cache_scale", ctypes.c_float * 4)]

    def __init__(self, h: int, d_h: int, R_K: int, R_V: int, dtype="bf16", rope_base: float = 1e4,
                 cache_format: int = 0, cache_scale=(0.0, 0.0, 0.0, 0.0)):
        if isinstance(dtype, str):
            dtype = {"bf16": TPA_BF16, "f32": TPA_F32}[dtype]
        elif isinstance(dtype, torch.dtype):
            dtype = {torch.bfloat16: TPA_BF16, torch.float32: TPA_F32}[dtype]
        if isinstance(cache_format, str):
            cache_format = {"native": TPA_CACHE_NATIVE, "e4m3": TPA_CACHE_E4M3}[cache_format]
        super().__init__(int(h), int(d_h), int(R_K), int(R_V), int(dtype), int(cache_format), float(rope_base),
                         (ctypes.c_float * 4)(*[float(x) for x in cache_scale]))

    @property
    def torch_dtype(self) -> torch.dtype:
        """Element type of factors and queries at the boundary."""
        return torch.bfloat16 if self.dtype == TPA_BF16 else torch.float32

    @property
    def cache_torch_dtype(self) -> torch.dtype:
        """Element type tpa_cache_read returns: uint8 codes for an E4M3 cache."""
        return torch.uint8 if self.cache_format == TPA_CACHE_E4M3 else self.torch_dtype

    def scale(self, k: int) -> float:
        """Stored-value scale of factor k (0 A_K, 1 B_K, 2 A_V, 3 B_V)."""
        if self.cache_format != TPA_CACHE_E4M3 or self.cache_scale[k] == 0.0:
            return 1.0
        return float(self.cache_scale[k])


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libtpa.so (built in-tree by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libtpa.so is not built ({_LIB_PATH}); run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _EXPORTS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _ref(d: Dims):
    return ctypes.byref(d)


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _numel(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """The C ABI takes bare pointers, so the binding checks element counts against the documented shapes
    before any launch: a short output would otherwise be written past its end."""
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n}")


def _cache_fits(dims: Dims, cache: torch.Tensor, capacity_tokens: int) -> None:
    need = tpa_cache_bytes(dims, capacity_tokens)
    if cache is not None and need > 0 and cache.numel() * cache.element_size() < need:
        raise ValueError(f"cache has {cache.numel() * cache.element_size()} bytes, a capacity of "
                         f"{capacity_tokens} tokens needs {need}")


def _factor_counts(dims: Dims, n: int, A_K, B_K, A_V, B_V) -> None:
    _numel(A_K, n * dims.R_K * dims.h, "A_K")
    _numel(B_K, n * dims.R_K * dims.d_h, "B_K")
    _numel(A_V, n * dims.R_V * dims.h, "A_V")
    _numel(B_V, n * dims.R_V * dims.d_h, "B_V")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, where: str):
    if status != 0:
        raise TPAError(status, where)


def tpa_abi_version() -> int:
    return int(load().tpa_abi_version())


def tpa_status_string(status: int) -> str:
    return load().tpa_status_string(int(status)).decode()


def tpa_supported(dims: Dims) -> bool:
    return bool(load().tpa_supported(_ref(dims)))


def tpa_block_tokens(dims: Dims) -> int:
    return int(load().tpa_block_tokens(_ref(dims)))


def tpa_cache_bytes(dims: Dims, capacity_tokens: int) -> int:
    return int(load().tpa_cache_bytes(_ref(dims), int(capacity_tokens)))


def tpa_decode_workspace_bytes(dims: Dims, batch: int, max_len: int, split_tokens: int = 0) -> int:
    return int(load().tpa_decode_workspace_bytes(_ref(dims), int(batch), int(max_len), int(split_tokens)))


def tpa_cache_append(dims: Dims, cache: torch.Tensor, capacity_tokens: int, slot: torch.Tensor,
                     kv_pos: torch.Tensor, A_K: torch.Tensor, B_K: torch.Tensor, A_V: torch.Tensor,
                     B_V: torch.Tensor, slot_hi: Optional[int] = None, q_pos: Optional[torch.Tensor] = None,
                     q_in: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    """Append factors of slot.numel() tokens (B_K rotated by kv_pos) and rotate optional query rows.

    A_K [n][R_K][h], B_K [n][R_K][d_h], A_V [n][R_V][h], B_V [n][R_V][d_h]; q_in/q_out [n_q][rows][d_h].
    ``slot_hi`` is a host-side bound on max(slot)+1 (default: capacity_tokens).
    """
    dt = dims.torch_dtype
    n_kv = slot.numel()
    n_q = 0 if q_pos is None else q_pos.numel()
    q_rows = 0
    if n_q:
        if q_in is None:
            raise ValueError("q_in is required with q_pos")
        q_out = q_in if q_out is None else q_out
        q_rows = q_in.numel() // (n_q * dims.d_h)
        _numel(q_in, max(q_rows, 1) * n_q * dims.d_h, "q_in")
        _numel(q_out, q_in.numel(), "q_out")
    _numel(kv_pos, n_kv, "kv_pos")
    _factor_counts(dims, n_kv, A_K, B_K, A_V, B_V)
    if n_kv:
        _cache_fits(dims, cache, capacity_tokens)
    lib = load()
    st = lib.tpa_cache_append(
        _ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), n_kv, _ptr(slot, torch.int64, "slot"),
        _ptr(kv_pos, torch.int32, "kv_pos"), int(capacity_tokens if slot_hi is None else slot_hi),
        _ptr(A_K, dt, "A_K"), _ptr(B_K, dt, "B_K"), _ptr(A_V, dt, "A_V"), _ptr(B_V, dt, "B_V"), n_q, q_rows,
        _ptr(q_pos, torch.int32, "q_pos") if n_q else None, _ptr(q_in, dt, "q_in") if n_q else None,
        _ptr(q_out, dt, "q_out") if n_q else None, _stream(stream))
    _check(st, "tpa_cache_append")


def tpa_cache_read(dims: Dims, cache: torch.Tensor, capacity_tokens: int, slot: torch.Tensor,
                   A_K: torch.Tensor, B_K: torch.Tensor, A_V: torch.Tensor, B_V: torch.Tensor, stream=None) -> None:
    """Stored factors of the given slots; uint8 E4M3 codes for an E4M3 cache."""
    dt = dims.cache_torch_dtype
    _factor_counts(dims, slot.numel(), A_K, B_K, A_V, B_V)
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_cache_read(_ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), slot.numel(),
                               _ptr(slot, torch.int64, "slot"), _ptr(A_K, dt, "A_K"), _ptr(B_K, dt, "B_K"),
                               _ptr(A_V, dt, "A_V"), _ptr(B_V, dt, "B_V"), _stream(stream))
    _check(st, "tpa_cache_read")


def tpa_decode(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
               seq_len: torch.Tensor, max_len: int, q_rot: torch.Tensor, out: torch.Tensor,
               workspace: torch.Tensor, scale: float = 0.0, split_tokens: int = 0, stream=None) -> None:
    """out[b][h][d_h] (fp32) = attention of q_rot[b] over the seq_len[b] cached tokens of sequence b."""
    batch = seq_start.numel()
    _numel(seq_len, batch, "seq_len")
    _numel(q_rot, batch * dims.h * dims.d_h, "q_rot")
    _numel(out, batch * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_decode(
        _ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(seq_len, torch.int32, "seq_len"), int(max_len),
        _ptr(q_rot, dims.torch_dtype, "q_rot"), float(scale), _ptr(out, torch.float32, "out"), int(split_tokens),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tpa_decode")


TPA_DECODE_NOALLOC_MAX_BYTES = 16 << 20  # the static partials array of tpa_decode_noalloc (tpa.h)


def tpa_decode_noalloc(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
                       seq_len: torch.Tensor, max_len: int, q_rot: torch.Tensor, out: torch.Tensor, scale: float = 0.0,
                       split_tokens: int = 0, stream=None) -> None:
    """tpa_decode with its partials in the library's static device array: no workspace, no allocation.
    Calls that overlap on one GPU race (they share the array)."""
    batch = seq_start.numel()
    _numel(seq_len, batch, "seq_len")
    _numel(q_rot, batch * dims.h * dims.d_h, "q_rot")
    _numel(out, batch * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_decode_noalloc(
        _ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(seq_len, torch.int32, "seq_len"), int(max_len),
        _ptr(q_rot, dims.torch_dtype, "q_rot"), float(scale), _ptr(out, torch.float32, "out"), int(split_tokens),
        _stream(stream))
    _check(st, "tpa_decode_noalloc")


def tpa_decode_step(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
                    seq_len: torch.Tensor, max_len: int, A_K: torch.Tensor, B_K: torch.Tensor, A_V: torch.Tensor,
                    B_V: torch.Tensor, q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                    scale: float = 0.0, split_tokens: int = 0, stream=None) -> None:
    """One fused decode step: append each sequence's new token at slot seq_start[b] + seq_len[b] (B_K rotated
    there), rotate q[b] at position seq_len[b], and write out[b] = attention over the seq_len[b] + 1 tokens."""
    dt = dims.torch_dtype
    batch = seq_start.numel()
    _numel(seq_len, batch, "seq_len")
    _factor_counts(dims, batch, A_K, B_K, A_V, B_V)
    _numel(q, batch * dims.h * dims.d_h, "q")
    _numel(out, batch * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_decode_step(
        _ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(seq_len, torch.int32, "seq_len"), int(max_len),
        _ptr(A_K, dt, "A_K"), _ptr(B_K, dt, "B_K"), _ptr(A_V, dt, "A_V"), _ptr(B_V, dt, "B_V"), _ptr(q, dt, "q"),
        float(scale), _ptr(out, torch.float32, "out"), int(split_tokens), _ptr(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tpa_decode_step")


def tpa_decode_fq(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
                  seq_len: torch.Tensor, max_len: int, A_Q: torch.Tensor, B_Q: torch.Tensor, out: torch.Tensor,
                  workspace: torch.Tensor, scale: float = 0.0, split_tokens: int = 0, stream=None) -> None:
    """Factored-query decode: q~[b][i] = RoPE at seq_len[b] of (1/R_Q) sum_r A_Q[b][r][i] B_Q[b][r], built on
    chip, then out[b] = attention over the seq_len[b] cached tokens.  A_Q [batch][R_Q][h], B_Q [batch][R_Q][d_h]
    (unrotated)."""
    dt = dims.torch_dtype
    batch = seq_start.numel()
    if A_Q.dim() != 3 or A_Q.shape[0] != batch or A_Q.shape[2] != dims.h:
        raise ValueError(f"A_Q must be [batch][R_Q][h] = [{batch}][R_Q][{dims.h}], got {list(A_Q.shape)}")
    _numel(seq_len, batch, "seq_len")
    _numel(B_Q, batch * A_Q.shape[1] * dims.d_h, "B_Q")
    _numel(out, batch * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_decode_fq(
        _ref(dims), int(A_Q.shape[1]), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(seq_len, torch.int32, "seq_len"), int(max_len),
        _ptr(A_Q, dt, "A_Q"), _ptr(B_Q, dt, "B_Q"), float(scale), _ptr(out, torch.float32, "out"),
        int(split_tokens), _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "tpa_decode_fq")


def tpa_prefill_chunk(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
                      ctx_len: torch.Tensor, max_ctx: int, chunk_len: int, q_rot: torch.Tensor, out: torch.Tensor,
                      scale: float = 0.0, stream=None) -> None:
    """out[b][j][h][d_h] (fp32): causal attention of chunk row j over slots 0 .. ctx_len[b] + j."""
    batch = seq_start.numel()
    _numel(ctx_len, batch, "ctx_len")
    _numel(q_rot, batch * chunk_len * dims.h * dims.d_h, "q_rot")
    _numel(out, batch * chunk_len * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_prefill_chunk(
        _ref(dims), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(ctx_len, torch.int32, "ctx_len"), int(max_ctx),
        int(chunk_len), _ptr(q_rot, dims.torch_dtype, "q_rot"), float(scale), _ptr(out, torch.float32, "out"),
        _stream(stream))
    _check(st, "tpa_prefill_chunk")


def tpa_prefill_chunk_fq(dims: Dims, cache: torch.Tensor, capacity_tokens: int, seq_start: torch.Tensor,
                         ctx_len: torch.Tensor, max_ctx: int, chunk_len: int, A_Q: torch.Tensor, B_Q: torch.Tensor,
                         out: torch.Tensor, scale: float = 0.0, stream=None) -> None:
    """Causal chunk with factored query rows: q~[b][j][i] = RoPE at ctx_len[b] + j of
    (1/R_Q) sum_r A_Q[b][j][r][i] B_Q[b][j][r], built on chip.  A_Q [batch][chunk][R_Q][h],
    B_Q [batch][chunk][R_Q][d_h] (unrotated)."""
    dt = dims.torch_dtype
    batch = seq_start.numel()
    if A_Q.dim() != 4 or A_Q.shape[0] != batch or A_Q.shape[1] != chunk_len or A_Q.shape[3] != dims.h:
        raise ValueError(f"A_Q must be [batch][chunk][R_Q][h] = [{batch}][{chunk_len}][R_Q][{dims.h}], "
                         f"got {list(A_Q.shape)}")
    _numel(ctx_len, batch, "ctx_len")
    _numel(B_Q, batch * chunk_len * A_Q.shape[2] * dims.d_h, "B_Q")
    _numel(out, batch * chunk_len * dims.h * dims.d_h, "out")
    _cache_fits(dims, cache, capacity_tokens)
    st = load().tpa_prefill_chunk_fq(
        _ref(dims), int(A_Q.shape[2]), _ptr(cache, name="cache"), int(capacity_tokens), seq_start.numel(),
        _ptr(seq_start, torch.int64, "seq_start"), _ptr(ctx_len, torch.int32, "ctx_len"), int(max_ctx),
        int(chunk_len), _ptr(A_Q, dt, "A_Q"), _ptr(B_Q, dt, "B_Q"), float(scale),
        _ptr(out, torch.float32, "out"), _stream(stream))
    _check(st, "tpa_prefill_chunk_fq")
