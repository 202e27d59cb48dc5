"""Shared set-up for the GPU parity tests: build a factor cache through the C ABI
from seeded inputs, run decode / prefill, and compare with the fp64 oracle.

Tolerances (element-wise over the whole output tensor), the stated ones:
  bf16 factors, fp32 accumulation: max-abs <= 1e-2 and rel-L2 <= 5e-3
  fp32 inputs:                     max-abs <= 1e-5 and rel-L2 <= 1e-5
Every case meets the rel-L2 bound.  A few stress cases (rank-1 factors, whose
outputs reach |5..10|, under a sharpened softmax or with few visible tokens)
exceed the max-abs bound; each is marked, with its measured error and the
cause, as an expected failure of that bound alone (``known_max_abs_excess``).
"""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np
import pytest
import torch

import factorized_kv_cache_tpa_amd as tpa
import oracle
import tpa_inputs as ti
from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device

TOL = {ti.BF16: (1e-2, 5e-3), ti.F32: (1e-5, 1e-5)}


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dims_of(w: ti.Workload, cache_format: int = 0, cache_scale=(0.0, 0.0, 0.0, 0.0)) -> tpa.Dims:
    return tpa.Dims(w.h, w.d_h, w.R_K, w.R_V, w.dtype, w.rope_base, cache_format, cache_scale)


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(gpu - ref) / den) if den > 0 else float(np.linalg.norm(gpu - ref))
    return max_abs, rel


class MaxAbsExceeded(AssertionError):
    """The output meets the rel-L2 bound but not the max-abs bound."""


def assert_close(gpu, ref, dtype: str, what: str = ""):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    max_abs, rel = errors(gpu, ref)
    tol_abs, tol_rel = TOL[dtype]
    say(f"  {what}: max_abs={max_abs:.3e} (bound {tol_abs:.1e}) rel_l2={rel:.3e} (bound {tol_rel:.1e})")
    assert rel <= tol_rel, f"{what}: rel_l2={rel:.3e} > {tol_rel:.1e} (max_abs={max_abs:.3e})"
    if max_abs > tol_abs:
        raise MaxAbsExceeded(f"{what}: max_abs={max_abs:.3e} > {tol_abs:.1e} (rel_l2={rel:.3e})")


class Checks:
    """Runs several assert_close checks and raises a max-abs excess only after all of them, so that every
    rel-L2 check of a test runs even where one comparison exceeds the max-abs bound."""

    def __init__(self):
        self.excess = []

    def close(self, gpu, ref, dtype: str, what: str = "") -> None:
        try:
            assert_close(gpu, ref, dtype, what)
        except MaxAbsExceeded as e:
            self.excess.append(str(e))

    def done(self) -> None:
        if self.excess:
            raise MaxAbsExceeded("; ".join(self.excess))


# Causes of the known max-abs excesses (the measured figures are in each test's table).
STORAGE_CAUSE = ("sharpened softmax over rank-1 factors (outputs up to |5..7|): the bf16 values of the rotated "
                 "B_K in the cache and of the rotated query row alone move the exact output by more than 1e-2 "
                 "(tests/test_storage_rounding.py shows it on the CPU, with no kernel involved); against exact "
                 "attention over those stored values the kernel is inside both bounds (the *_stored_values tests)")


def stored_key_and_query(B_K: np.ndarray, q: np.ndarray, q_pos, w: ti.Workload, dims: tpa.Dims):
    """B_K [n][R][d] and query rows q [rows][h][d] (at positions q_pos) replaced by the values the kernel
    reads.  bf16 only: an E4M3 B_K is a stored value already (stored_factors), only the query is rounded."""
    assert w.dtype == ti.BF16
    if dims.cache_format != tpa.TPA_CACHE_E4M3:
        B_K = stored_rotated(B_K, np.arange(B_K.shape[0], dtype=np.float64)[:, None], w.rope_base)
    q = stored_rotated(q, np.asarray(q_pos, dtype=np.float64).reshape(-1, 1), w.rope_base)
    return B_K, q


def stored_rotated(x: np.ndarray, pos, base: float) -> np.ndarray:
    """What a bf16 buffer of x's rows rotated to pos holds (pos: one per row, broadcast), rotated back in fp64,
    so the oracle, which rotates whole rows itself, sees exactly the stored rotated values.  Oracle side only."""
    pos = np.asarray(pos, dtype=np.float64)
    return oracle.rope_rows_at(oracle.round_to_bf16(oracle.rope_rows_at(x, pos, base)), -pos, base)


def known_max_abs_excess(request, measured: str, cause: str) -> None:
    """Mark the running test as an expected failure of the max-abs bound alone: a rel-L2 miss, a non-finite
    output or any other error still fails it, and so does a pass (strict), so the list stays current."""
    request.applymarker(pytest.mark.xfail(raises=MaxAbsExceeded, strict=True,
                                          reason=f"measured {measured}; cause: {cause}"))


def f64(a, dtype):
    return ti.to_f64(a, dtype)


class DecodeSetup:
    """Cache + rotated queries for a batch of decode sequences."""

    def __init__(self, w: ti.Workload, seqs: Sequence[ti.Sequence], lens: Optional[Sequence[int]] = None,
                 extra_capacity: int = 0, q_positions: Optional[Sequence[int]] = None,
                 dims: Optional[tpa.Dims] = None):
        self.w = w
        self.dims = dims_of(w) if dims is None else dims
        self.seqs = list(seqs)
        self.lens = [s.n_tokens for s in self.seqs] if lens is None else list(lens)
        self.cache = FactorCache(self.dims, [n + extra_capacity for n in self.lens])
        for b, s in enumerate(self.seqs):
            if s.n_tokens:
                self.cache.append_host(b, s.A_K, s.B_K, s.A_V, s.B_V)
        q = np.stack([s.q[0] for s in self.seqs])  # [batch][h][d]
        q_dev = to_device(q, self.dims)
        self.q_positions = list(self.lens if q_positions is None else q_positions)
        q_pos = torch.tensor(self.q_positions, dtype=torch.int32, device="cuda")
        self.q_rot = self.cache.rotate_queries(q_dev, q_pos)
        self.seq_len = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.batch = len(self.seqs)
        self.max_len = max(self.lens) if self.lens else 0

    def run(self, split_tokens: int = 0, scale: float = 0.0, seq_start: Optional[torch.Tensor] = None,
            seq_len: Optional[torch.Tensor] = None, max_len: Optional[int] = None,
            capacity: Optional[int] = None) -> np.ndarray:
        """capacity: the capacity the call declares (default the cache's own)."""
        max_len = self.max_len if max_len is None else max_len
        ws_bytes = tpa.tpa_decode_workspace_bytes(self.dims, self.batch, max_len, split_tokens)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        out = torch.full((self.batch, self.w.h, self.w.d_h), float("nan"), dtype=torch.float32, device="cuda")
        tpa.tpa_decode(self.dims, self.cache.buf, self.cache.capacity if capacity is None else capacity,
                       self.cache.seq_start if seq_start is None else seq_start,
                       self.seq_len if seq_len is None else seq_len, max_len, self.q_rot, out, ws, scale=scale,
                       split_tokens=split_tokens)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def factors(self, b: int, n: int):
        """The cached factor values the oracle attends over (fp64)."""
        return stored_factors(self.seqs[b], n, self.w, self.dims)

    def oracle(self, b: int, scale: Optional[float] = None, as_stored: bool = False) -> np.ndarray:
        """as_stored: over the values the kernel reads (the query rotated and rounded to bf16; in a native
        cache also B_K rotated and rounded per token) instead of the caller's factors."""
        s, dt = self.seqs[b], self.w.dtype
        n = self.lens[b]
        A_K, B_K, A_V, B_V = self.factors(b, n)
        q = f64(s.q[:1], dt)
        if as_stored:
            B_K, q = stored_key_and_query(B_K, q, self.q_positions[b], self.w, self.dims)
        return oracle.attention(A_K, B_K, A_V, B_V, np.arange(n), q, [self.q_positions[b]], [n],
                                self.w.rope_base, scale)[0]


class PrefillSetup:
    """Cache holding ctx + chunk tokens per sequence, rotated chunk query rows."""

    def __init__(self, w: ti.Workload, seqs: Sequence[ti.Sequence], ctx: Sequence[int],
                 dims: Optional[tpa.Dims] = None, extra_capacity: int = 0):
        self.w = w
        self.dims = dims_of(w) if dims is None else dims
        self.seqs = list(seqs)
        self.ctx = list(ctx)
        self.chunk = self.seqs[0].q.shape[0]
        assert all(s.q.shape[0] == self.chunk for s in self.seqs)
        assert all(s.n_tokens == c + self.chunk for s, c in zip(self.seqs, self.ctx))
        self.cache = FactorCache(self.dims, [s.n_tokens + extra_capacity for s in self.seqs])
        for b, s in enumerate(self.seqs):
            self.cache.append_host(b, s.A_K, s.B_K, s.A_V, s.B_V)
        q = np.stack([s.q for s in self.seqs])  # [batch][chunk][h][d]
        q_dev = to_device(q, self.dims).reshape(len(self.seqs) * self.chunk, self.w.h, self.w.d_h)
        q_pos = torch.tensor(np.concatenate([c + np.arange(self.chunk) for c in self.ctx]), dtype=torch.int32,
                             device="cuda")
        self.q_rot = self.cache.rotate_queries(q_dev, q_pos).reshape(len(self.seqs), self.chunk, self.w.h,
                                                                      self.w.d_h)
        self.ctx_len = torch.tensor(self.ctx, dtype=torch.int32, device="cuda")

    def run(self, scale: float = 0.0, seq_start=None, capacity: Optional[int] = None) -> np.ndarray:
        """capacity: the capacity the call declares (default the cache's own)."""
        out = torch.full((len(self.seqs), self.chunk, self.w.h, self.w.d_h), float("nan"), dtype=torch.float32,
                         device="cuda")
        starts = self.cache.seq_start if seq_start is None else seq_start
        cap = self.cache.capacity if capacity is None else capacity
        tpa.tpa_prefill_chunk(self.dims, self.cache.buf, cap, starts, self.ctx_len,
                              max(self.ctx), self.chunk, self.q_rot, out, scale=scale)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, b: int, rows=None, as_stored: bool = False) -> np.ndarray:
        """as_stored: over the values the kernel reads (B_K rotated and rounded to bf16 per token, query rows
        rotated and rounded per row) instead of the caller's factors; the other factors are exact either way."""
        s, dt = self.seqs[b], self.w.dtype
        A_K, B_K, A_V, B_V = stored_factors(s, s.n_tokens, self.w, self.dims)
        q = f64(s.q, dt)
        if as_stored:
            B_K, q = stored_key_and_query(B_K, q, self.ctx[b] + np.arange(self.chunk), self.w, self.dims)
        return oracle.prefill(A_K, B_K, A_V, B_V, q, self.ctx[b], self.w.rope_base, rows=rows)


def e4m3_values(x: np.ndarray, scale: float) -> np.ndarray:
    """Stored values of an E4M3 cache: code = E4M3(x / scale), value = code * scale (the oracle's codec)."""
    return oracle.e4m3_decode(oracle.e4m3_encode(np.asarray(x, dtype=np.float64) / scale)) * scale


def stored_factors(s: ti.Sequence, n: int, w: ti.Workload, dims: tpa.Dims):
    """The first n tokens' factors as the cache holds them, in fp64, computed on the oracle side only.
    Native cache: the inputs.  E4M3 cache: every factor through the oracle's codec; B_K is stored rotated
    (RoPE on B only), so its stored value is rotated back to the token's position 0 frame, and the
    oracle, which rotates whole key rows itself, sees exactly the stored key."""
    dt = w.dtype
    A_K, B_K, A_V, B_V = (f64(x[:n], dt) for x in (s.A_K, s.B_K, s.A_V, s.B_V))
    if dims.cache_format != tpa.TPA_CACHE_E4M3:
        return A_K, B_K, A_V, B_V
    A_K, A_V, B_V = e4m3_values(A_K, dims.scale(0)), e4m3_values(A_V, dims.scale(2)), e4m3_values(B_V, dims.scale(3))
    if n:
        pos = np.arange(n, dtype=np.float64)[:, None]  # token t's rank rows sit at position t
        B_K = oracle.rope_rows_at(e4m3_values(oracle.rope_rows_at(B_K, pos, w.rope_base), dims.scale(1)), -pos,
                                  w.rope_base)
    return A_K, B_K, A_V, B_V


def case_workload(h, d_h, R_K, R_V, dtype=ti.BF16, base=1e4, seed=7) -> ti.Workload:
    return ti.custom("case", seed, h, d_h, R_K, R_V, dtype, base, 1)


def random_sequences(w: ti.Workload, lens: List[int], n_q: int = 1, q_scale: float = 1.0, seed: int = 0):
    ss = np.random.SeedSequence(seed).spawn(len(lens))
    return [ti.draw_sequence(ss[i], n, n_q, w, q_scale) for i, n in enumerate(lens)]
