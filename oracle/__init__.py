"""fp64 CPU oracle for attention over a TPA factor cache.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  The library
(``factorized_kv_cache_tpa_amd``) never imports it and shares no code with it.

The arithmetic lives in ``tpa_oracle.c`` (plain C, fp64, OpenMP over heads):
materialize K and V from the factors, apply standard RoPE to the full key and
query rows, run textbook two-pass softmax attention.  This wrapper only
marshals numpy arrays and maps decode / prefill onto that one routine:

* decode (one query row per sequence at position N, sees all N cached tokens);
* causal chunked prefill (chunk row j at position ctx + j sees tokens
  0 .. ctx + j, including the chunk's own earlier tokens and itself).

The reading of the pages these follow is spelled out in ``tpa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tpa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        D = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.POINTER(ctypes.c_int64)
        lib.tpa_oracle_rope_row.argtypes = [D, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        lib.tpa_oracle_rope_row.restype = None
        lib.tpa_oracle_rope_rows.argtypes = [D, ctypes.c_int64, ctypes.c_int, D, ctypes.c_double, ctypes.c_int]
        lib.tpa_oracle_rope_rows.restype = None
        lib.tpa_oracle_attention.argtypes = [ctypes.c_int] * 4 + [ctypes.c_int64] + [D] * 5 + [
            ctypes.c_int64, D, D, I64, ctypes.c_double, ctypes.c_double, D, ctypes.c_int]
        lib.tpa_oracle_attention.restype = ctypes.c_int
        lib.tpa_oracle_query_from_factors.argtypes = [ctypes.c_int] * 3 + [ctypes.c_int64, D, D, D]
        lib.tpa_oracle_query_from_factors.restype = None
        lib.tpa_oracle_factor_elems_per_token.argtypes = [ctypes.c_int] * 4
        lib.tpa_oracle_factor_elems_per_token.restype = ctypes.c_int64
        lib.tpa_oracle_dense_elems_per_token.argtypes = [ctypes.c_int] * 2
        lib.tpa_oracle_dense_elems_per_token.restype = ctypes.c_int64
        lib.tpa_oracle_max_threads.restype = ctypes.c_int
        U8 = ctypes.POINTER(ctypes.c_uint8)
        lib.tpa_oracle_e4m3_decode_n.argtypes = [ctypes.c_int64, U8, D]
        lib.tpa_oracle_e4m3_encode_n.argtypes = [ctypes.c_int64, D, U8]
        _lib = lib
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def max_threads() -> int:
    return int(_load().tpa_oracle_max_threads())


def rope_rows(x: np.ndarray, pos: float, base: float) -> np.ndarray:
    """Standard RoPE of every last-axis row of x (even length) at one position; returns a copy."""
    y = _f64(x).copy()
    flat = y.reshape(-1, y.shape[-1])
    lib = _load()
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib.tpa_oracle_rope_row(_dp(row), int(row.shape[0]), float(pos), float(base))
        flat[r] = row
    return y


def rope_rows_at(x: np.ndarray, pos, base: float, threads: Optional[int] = None) -> np.ndarray:
    """Standard RoPE of every last-axis row of x at its own position: pos has the shape of x without the last
    axis (or broadcasts to it).  Each row is rotated exactly as rope_rows rotates it; returns a copy."""
    y = _f64(x).copy()
    d = y.shape[-1]
    p = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.float64), y.shape[:-1]))
    n = int(np.prod(y.shape[:-1]))
    _load().tpa_oracle_rope_rows(_dp(y), n, int(d), _dp(p), float(base),
                                 int(threads if threads is not None else max_threads()))
    return y


def attention(A_K, B_K, A_V, B_V, kv_pos, q, q_pos, q_nvis, base: float, scale: Optional[float] = None,
              threads: Optional[int] = None) -> np.ndarray:
    """out[n][h][d] for query rows q[n][h][d] over cached factors (all float64-convertible)."""
    A_K, B_K, A_V, B_V = _f64(A_K), _f64(B_K), _f64(A_V), _f64(B_V)
    q = _f64(q)
    n_kv, RK, h = A_K.shape
    RV = A_V.shape[1]
    d = B_K.shape[2]
    n_q = q.shape[0]
    assert B_K.shape == (n_kv, RK, d) and A_V.shape == (n_kv, RV, h) and B_V.shape == (n_kv, RV, d)
    assert q.shape == (n_q, h, d)
    kv_pos = _f64(kv_pos).reshape(n_kv)
    q_pos = _f64(q_pos).reshape(n_q)
    q_nvis = np.ascontiguousarray(q_nvis, dtype=np.int64).reshape(n_q)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n_q, h, d), dtype=np.float64)
    nt = threads if threads is not None else max_threads()
    rc = _load().tpa_oracle_attention(
        h, d, RK, RV, n_kv, _dp(A_K), _dp(B_K), _dp(A_V), _dp(B_V), _dp(kv_pos), n_q, _dp(q), _dp(q_pos),
        q_nvis.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), float(base), float(scale), _dp(out), int(nt))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def query_from_factors(A_Q, B_Q) -> np.ndarray:
    """Query rows from query factors: q[n][i][c] = (1/R_Q) sum_r A_Q[n][r][i] B_Q[n][r][c] -> [n][h][d]."""
    A_Q, B_Q = _f64(A_Q), _f64(B_Q)
    n, RQ, h = A_Q.shape
    d = B_Q.shape[2]
    assert B_Q.shape == (n, RQ, d)
    out = np.zeros((n, h, d), dtype=np.float64)
    _load().tpa_oracle_query_from_factors(h, d, RQ, n, _dp(A_Q), _dp(B_Q), _dp(out))
    return out


def decode(A_K, B_K, A_V, B_V, q, base: float, scale: Optional[float] = None, n_cached: Optional[int] = None,
           threads: Optional[int] = None) -> np.ndarray:
    """One query row q[h][d] at position N over N cached tokens at positions 0..N-1 -> [h][d]."""
    n = int(np.shape(A_K)[0]) if n_cached is None else int(n_cached)
    q = _f64(q).reshape((1,) + np.shape(q)[-2:])
    return attention(A_K, B_K, A_V, B_V, np.arange(np.shape(A_K)[0]), q, [n], [n], base, scale, threads)[0]


def prefill(A_K, B_K, A_V, B_V, q, ctx: int, base: float, scale: Optional[float] = None,
            rows: Optional[np.ndarray] = None, threads: Optional[int] = None) -> np.ndarray:
    """Causal chunk: query row j at position ctx+j sees tokens 0..ctx+j -> [n_rows][h][d].

    ``rows`` selects a subset of chunk rows (sampled checks); default all rows of q.
    """
    q = _f64(q)
    j = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    return attention(A_K, B_K, A_V, B_V, np.arange(np.shape(A_K)[0]), q[j], ctx + j, ctx + j + 1, base,
                     scale, threads)


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> their values in fp64 (NaN for S.1111.111)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().tpa_oracle_e4m3_decode_n(c.size, c.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _dp(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    """fp64 values -> nearest OCP E4M3 codes (ties to even, saturating at +-448)."""
    v = _f64(x)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().tpa_oracle_e4m3_encode_n(v.size, _dp(v), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    return out


def round_to_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each fp64 value, ties to even (returned as fp64).  The storage format of a bf16
    cache: 8 significant bits, the fp32 exponent range.  Computed as round-to-odd to fp32 (truncate, then set
    the last bit when inexact), which keeps the two guard bits that the final round to nearest even needs,
    so the result equals a direct rounding of x.  Finite inputs inside the fp32 range."""
    v = _f64(x)
    t = v.astype(np.float32)
    # truncate toward zero: step back one fp32 unit where the fp32 rounding went past |x|
    over = np.abs(t.astype(np.float64)) > np.abs(v)
    t = np.where(over, np.nextafter(t, np.float32(0)), t)
    bits = t.view(np.uint32).copy()
    inexact = t.astype(np.float64) != v
    bits |= inexact.astype(np.uint32)  # round to odd
    rne = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return rne.view(np.float32).astype(np.float64)


def factor_elems_per_token(h: int, d: int, RK: int, RV: int) -> int:
    return int(_load().tpa_oracle_factor_elems_per_token(h, d, RK, RV))


def dense_elems_per_token(h: int, d: int) -> int:
    return int(_load().tpa_oracle_dense_elems_per_token(h, d))
