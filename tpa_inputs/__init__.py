"""Seeded synthetic inputs for attention over a TPA factor cache.

This module only draws random numbers and converts storage formats. It holds
none of the method's arithmetic (no RoPE, no factor products, no softmax), so
both the fp64 CPU oracle and the HIP path can take their inputs from here
without sharing any computation.

Recipe (the same for every workload):
  * numpy ``Generator(PCG64(seed))``; every sequence gets its own child
    generator from ``SeedSequence(seed).spawn(...)`` so any one sequence can be
    regenerated alone (the oracle checks sampled sequences of the large
    workloads that way).
  * per sequence, in this order: A_K [N][R_K][h], B_K [N][R_K][d_h],
    A_V [N][R_V][h], B_V [N][R_V][d_h], each ``standard_normal(float32)`` times
    1/sqrt(R) (variance 1/R), then the query rows q [n_q][h][d_h] times
    1/sqrt(d_h) (variance 1/d_h).  Factors are i.i.d. Gaussian with no
    structure.
  * bf16 workloads round the float32 draws to bf16 by round-to-nearest-even;
    fp32 workloads keep the float32 draws.  Arrays are returned in storage
    form: ``uint16`` bit patterns for bf16, ``float32`` for fp32.
  * factors are *unrotated*; cached token j of a sequence sits at position j,
    a decode query at position N (the number of cached tokens), prefill chunk
    row j at position ctx + j.

Workload names describe the shapes; the definitions mirror the five
configurations the library is measured on (tiny fp32 decode; two bf16 decode
batches; a 131072-token decode; a ragged decode batch plus a causal prefill
chunk).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    h: int
    d_h: int
    R_K: int
    R_V: int
    dtype: str
    rope_base: float
    batch: int
    # decode: cached tokens per sequence (fixed) or None when ragged
    n_cached: Optional[int] = None
    ragged_lo: Optional[int] = None
    ragged_hi: Optional[int] = None
    # prefill part (ragged + prefill workload only)
    prefill_batch: int = 0
    prefill_ctx: int = 0
    prefill_chunk: int = 0


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_decode_b1_h4_d16_r1_n64_f32", 1001, 4, 16, 1, 1, F32, 1e4, 1, n_cached=64),
        Workload("decode_b16_h32_d128_r1_n4096", 1002, 32, 128, 1, 1, BF16, 1e4, 16, n_cached=4096),
        Workload("decode_b64_h16_d64_r2_n8192", 1003, 16, 64, 2, 2, BF16, 1e4, 64, n_cached=8192),
        Workload("longctx_decode_b4_h32_d128_r2_n131072", 1004, 32, 128, 2, 2, BF16, 5e5, 4,
                 n_cached=131072),
        Workload("ragged_decode_b128_h32_d128_r4_plus_prefill_b8_ctx2048_chunk512", 1005, 32, 128, 4, 4,
                 BF16, 1e4, 128, ragged_lo=1024, ragged_hi=32768,
                 prefill_batch=8, prefill_ctx=2048, prefill_chunk=512),
    ]
}

# short names: what sets each workload apart
ALIASES = {
    "tiny": "tiny_decode_b1_h4_d16_r1_n64_f32",
    "rank1": "decode_b16_h32_d128_r1_n4096",
    "h16": "decode_b64_h16_d64_r2_n8192",
    "longctx": "longctx_decode_b4_h32_d128_r2_n131072",
    "ragged": "ragged_decode_b128_h32_d128_r4_plus_prefill_b8_ctx2048_chunk512",
}
assert set(ALIASES.values()) == set(WORKLOADS)


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def custom(name: str, seed: int, h: int, d_h: int, R_K: int, R_V: int, dtype: str,
           rope_base: float, batch: int, n_cached: Optional[int] = None, **kw) -> Workload:
    """A workload of arbitrary shape (small parity cases and edge cases)."""
    return Workload(name, seed, h, d_h, R_K, R_V, dtype, rope_base, batch, n_cached=n_cached, **kw)


# ----------------------------------------------------------------------------------------------
# storage conversions (exact; no method arithmetic)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact promotion of a storage-form array to float64."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32)


# ----------------------------------------------------------------------------------------------
# generation

def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    return to_storage(x, dtype)


@dataclasses.dataclass
class Sequence:
    """One sequence's inputs in storage form (see module docstring)."""
    A_K: np.ndarray
    B_K: np.ndarray
    A_V: np.ndarray
    B_V: np.ndarray
    q: np.ndarray  # [n_q][h][d_h]

    @property
    def n_tokens(self) -> int:
        return int(self.A_K.shape[0])


def draw_sequence(seed_seq: np.random.SeedSequence, n_tokens: int, n_q: int, w: Workload,
                  q_scale: float = 1.0) -> Sequence:
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    sk, sv = 1.0 / np.sqrt(w.R_K), 1.0 / np.sqrt(w.R_V)
    A_K = _draw(rng, (n_tokens, w.R_K, w.h), sk, w.dtype)
    B_K = _draw(rng, (n_tokens, w.R_K, w.d_h), sk, w.dtype)
    A_V = _draw(rng, (n_tokens, w.R_V, w.h), sv, w.dtype)
    B_V = _draw(rng, (n_tokens, w.R_V, w.d_h), sv, w.dtype)
    q = _draw(rng, (n_q, w.h, w.d_h), q_scale / np.sqrt(w.d_h), w.dtype)
    return Sequence(A_K, B_K, A_V, B_V, q)


def decode_lengths(w: Workload) -> np.ndarray:
    """Cached length of every decode sequence (ragged workloads draw them first)."""
    if w.n_cached is not None:
        return np.full(w.batch, w.n_cached, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed).spawn(1)[0]))
    return rng.integers(w.ragged_lo, w.ragged_hi, size=w.batch, endpoint=True).astype(np.int64)


def _children(w: Workload):
    # child 0: lengths; children 1..batch: decode sequences; then the prefill sequences
    return np.random.SeedSequence(w.seed).spawn(1 + w.batch + w.prefill_batch)


def decode_sequence(w: Workload, b: int, q_scale: float = 1.0) -> Sequence:
    """Decode sequence b: its cached factors (positions 0..N-1) and one query row (position N)."""
    n = int(decode_lengths(w)[b])
    return draw_sequence(_children(w)[1 + b], n, 1, w, q_scale)


def prefill_sequence(w: Workload, p: int, q_scale: float = 1.0) -> Sequence:
    """Prefill sequence p: ctx + chunk tokens of factors and chunk query rows."""
    return draw_sequence(_children(w)[1 + w.batch + p], w.prefill_ctx + w.prefill_chunk,
                         w.prefill_chunk, w, q_scale)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def decode_batch(w: Workload, q_scale: float = 1.0, only: Optional[List[int]] = None) -> List[Sequence]:
    idx = list(range(w.batch)) if only is None else list(only)
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        return list(ex.map(lambda b: decode_sequence(w, b, q_scale), idx))


def prefill_batch(w: Workload, q_scale: float = 1.0) -> List[Sequence]:
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        return list(ex.map(lambda p: prefill_sequence(w, p, q_scale), range(w.prefill_batch)))


def random_case(seed: int, n_tokens: int, n_q: int, h: int, d_h: int, R_K: int, R_V: int,
                dtype: str = F32, q_scale: float = 1.0) -> Sequence:
    """A single sequence of arbitrary shape for small parity and edge cases."""
    w = custom("case", seed, h, d_h, R_K, R_V, dtype, 1e4, 1)
    return draw_sequence(np.random.SeedSequence(seed), n_tokens, n_q, w, q_scale)
