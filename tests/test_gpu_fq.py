"""GPU parity of the factored-query decode (tpa_decode_fq) and prefill (tpa_prefill_chunk_fq) against the
fp64 oracle.

The query arrives as factors (A_Q [R_Q][h], B_Q [R_Q][d_h], unrotated); the library builds
q = (1/R_Q) A_Q^T B_Q on chip, rotates it at the query's position (the cached length for decode,
ctx + j for prefill row j) and rounds it once.  The oracle builds q = (1/R_Q) A_Q^T B_Q in fp64
(oracle.query_from_factors, pinned on the CPU) and rotates the full query row at the same position.
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_tpa_amd as tpa
import oracle
import tpa_inputs as ti
from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device
from tests.gpu_cases import (STORAGE_CAUSE, Checks, assert_close, case_workload, dims_of, f64,
                             known_max_abs_excess, random_sequences, say, stored_rotated)

pytestmark = pytest.mark.gpu


class FQSetup:
    def __init__(self, w: ti.Workload, lens, R_Q: int, q_scale: float = 1.0, seed: int = 0, seqs=None):
        self.w, self.dims, self.lens, self.R_Q = w, dims_of(w), list(lens), R_Q
        self.seqs = seqs if seqs is not None else random_sequences(w, lens, seed=seed)
        self.cache = FactorCache(self.dims, self.lens)
        for b, (s, n) in enumerate(zip(self.seqs, self.lens)):
            if n:
                self.cache.append_host(b, s.A_K[:n], s.B_K[:n], s.A_V[:n], s.B_V[:n])
        rng = np.random.default_rng(seed + 1000 * R_Q)
        B = len(self.lens)
        # query factors: N(0, 1) head factor, N(0, q_scale^2 / d_h) feature factor, rounded to storage
        self.A_Q = ti.to_storage(rng.standard_normal((B, R_Q, w.h), dtype=np.float32), w.dtype)
        self.B_Q = ti.to_storage(rng.standard_normal((B, R_Q, w.d_h), dtype=np.float32) * (q_scale / np.sqrt(w.d_h)),
                                 w.dtype)
        self.seq_len = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.A_Q_dev = to_device(self.A_Q, self.dims)
        self.B_Q_dev = to_device(self.B_Q, self.dims)  # the query sits at position N (the kernel rotates it)
        self.batch, self.max_len = B, max(self.lens)

    def run(self, split_tokens: int = 0) -> np.ndarray:
        ws = torch.zeros(max(256, tpa.tpa_decode_workspace_bytes(self.dims, self.batch, self.max_len, split_tokens)),
                         dtype=torch.uint8, device="cuda")
        out = torch.full((self.batch, self.w.h, self.w.d_h), float("nan"), dtype=torch.float32, device="cuda")
        tpa.tpa_decode_fq(self.dims, self.cache.buf, self.cache.capacity, self.cache.seq_start, self.seq_len,
                          self.max_len, self.A_Q_dev, self.B_Q_dev, out, ws, split_tokens=split_tokens)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle(self, b: int) -> np.ndarray:
        s, n, dt = self.seqs[b], self.lens[b], self.w.dtype
        q = oracle.query_from_factors(f64(self.A_Q[b:b + 1], dt), f64(self.B_Q[b:b + 1], dt))[0]
        return oracle.decode(f64(s.A_K[:n], dt), f64(s.B_K[:n], dt), f64(s.A_V[:n], dt), f64(s.B_V[:n], dt), q,
                             self.w.rope_base)


CASES = [(32, 128, 1, 1, ti.BF16, 1e4, 1), (32, 128, 1, 1, ti.BF16, 1e4, 6), (32, 128, 2, 2, ti.BF16, 5e5, 16),
         (16, 64, 2, 2, ti.BF16, 1e4, 3), (20, 48, 1, 3, ti.BF16, 1e4, 2), (4, 16, 1, 1, ti.F32, 1e4, 2),
         (32, 128, 3, 2, ti.F32, 5e5, 16), (64, 64, 2, 2, ti.BF16, 1e4, 4), (64, 64, 1, 1, ti.BF16, 1e4, 4), (56, 32, 2, 2, ti.BF16, 1e4, 5),
         (16, 128, 2, 2, ti.F32, 1e4, 3)]


# Sharpened rank-1 cases whose max-abs error exceeds 1e-2 (measured on MI355X; rel-L2 within 5e-3).
SHARP_RANK1 = {}


@pytest.mark.parametrize("h,d_h,R_K,R_V,dtype,base,R_Q", CASES)
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_fq_matches_oracle(h, d_h, R_K, R_V, dtype, base, R_Q, q_scale, request):
    w = case_workload(h, d_h, R_K, R_V, dtype, base)
    lens = [1, 31, 32, 33, 300, 1000]
    known = SHARP_RANK1.get((h, d_h, R_K, R_V, R_Q, q_scale))
    if known:
        known_max_abs_excess(request, known, STORAGE_CAUSE)
    say(f"case: fq h={h} d_h={d_h} R_K={R_K} R_V={R_V} R_Q={R_Q} {dtype} q_scale={q_scale}")
    st = FQSetup(w, lens, R_Q, q_scale=q_scale, seed=h + d_h + R_Q)
    got = st.run()
    chk = Checks()
    for b in range(st.batch):
        chk.close(got[b], st.oracle(b), dtype, f"seq {b} (N={lens[b]})")
    chk.done()


def test_fq_with_identity_head_factor_equals_plain_decode():
    """R_Q = h and A_Q = R_Q * I: the built query is exactly the B_Q rows (h x b / h = b in fp32 for bf16 b and
    h a power of two, and scaling by a power of two commutes with the fp32 rotation), so the output equals
    tpa_decode with q = the B_Q rows rotated by tpa_cache_append at the same position, bit for bit."""
    w = case_workload(32, 128, 1, 1, ti.BF16)
    st = FQSetup(w, [100, 2500], R_Q=32, seed=4)
    eye = np.broadcast_to(np.eye(32, dtype=np.float32) * 32.0, (2, 32, 32))
    st.A_Q = ti.to_storage(eye, ti.BF16)
    st.A_Q_dev = to_device(st.A_Q, st.dims)
    with pytest.raises(tpa.TPAError):  # R_Q = 32 is past the supported rank; check the guard, then use 16
        st.run()
    st = FQSetup(case_workload(16, 128, 1, 1, ti.BF16), [100, 2500], R_Q=16, seed=4)
    eye = np.broadcast_to(np.eye(16, dtype=np.float32) * 16.0, (2, 16, 16))
    st.A_Q = ti.to_storage(eye, ti.BF16)
    st.A_Q_dev = to_device(st.A_Q, st.dims)
    got = st.run()
    ws = torch.zeros(tpa.tpa_decode_workspace_bytes(st.dims, st.batch, st.max_len), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(st.batch, 16, 128, dtype=torch.float32, device="cuda")
    q_rot = st.cache.rotate_queries(st.B_Q_dev, st.seq_len)
    tpa.tpa_decode(st.dims, st.cache.buf, st.cache.capacity, st.cache.seq_start, st.seq_len, st.max_len,
                   q_rot, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, out.cpu().numpy())


@pytest.mark.parametrize("split_tokens", [32, 256, 4096])
def test_fq_split_sizes(split_tokens):
    w = case_workload(32, 128, 2, 2, ti.BF16)
    st = FQSetup(w, [5, 700, 2100], R_Q=6, q_scale=8.0, seed=17)
    got = st.run(split_tokens=split_tokens)
    for b in range(st.batch):
        assert_close(got[b], st.oracle(b), ti.BF16, f"split {split_tokens} seq {b}")


def test_fq_full_size_decode_b16_h32_d128_r1_n4096_rq6():
    """The metric's cache (16 x 4096 cached tokens, h=32, d_h=128, R=1) with a rank-6 factored query,
    every sequence checked."""
    w = ti.get("rank1")
    say(f"case: fq full size {w.name} R_Q=6")
    lens = list(ti.decode_lengths(w))
    st = FQSetup(w, lens, R_Q=6, seqs=ti.decode_batch(w), seed=w.seed)
    got = st.run()
    for b in range(st.batch):
        assert_close(got[b], st.oracle(b), w.dtype, f"seq {b}")


def _prefill_fq_case(h, d_h, R_K, R_V, R_Q, ctxs, chunk, as_stored=False):
    """Run tpa_prefill_chunk_fq on seeded inputs; compare every row with the oracle on the factors, or
    (as_stored) on the values the kernel reads: B_K rotated and rounded to bf16 per token, and each query row
    built from its factors, rotated and rounded once to bf16."""
    w = case_workload(h, d_h, R_K, R_V, ti.BF16)
    dims = dims_of(w)
    seqs = random_sequences(w, [c + chunk for c in ctxs], seed=h + R_Q)
    cache = FactorCache(dims, [c + chunk for c in ctxs])
    for b, s in enumerate(seqs):
        cache.append_host(b, s.A_K, s.B_K, s.A_V, s.B_V)
    rng = np.random.default_rng(R_Q * 31 + chunk)
    B = len(ctxs)
    A_Q = ti.to_storage(rng.standard_normal((B, chunk, R_Q, h), dtype=np.float32), ti.BF16)
    B_Q = ti.to_storage(rng.standard_normal((B, chunk, R_Q, d_h), dtype=np.float32) * (4.0 / np.sqrt(d_h)), ti.BF16)
    out = torch.full((B, chunk, h, d_h), float("nan"), dtype=torch.float32, device="cuda")
    tpa.tpa_prefill_chunk_fq(dims, cache.buf, cache.capacity, cache.seq_start,
                             torch.tensor(ctxs, dtype=torch.int32, device="cuda"), max(ctxs), chunk,
                             to_device(A_Q, dims), to_device(B_Q, dims), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    chk = Checks()
    for b, s in enumerate(seqs):
        q = oracle.query_from_factors(f64(A_Q[b], ti.BF16), f64(B_Q[b], ti.BF16))
        B_K = f64(s.B_K, ti.BF16)
        if as_stored:
            n = B_K.shape[0]
            B_K = stored_rotated(B_K, np.arange(n, dtype=np.float64)[:, None], w.rope_base)
            q = stored_rotated(q, (ctxs[b] + np.arange(chunk, dtype=np.float64))[:, None], w.rope_base)
        ref = oracle.prefill(f64(s.A_K, ti.BF16), B_K, f64(s.A_V, ti.BF16), f64(s.B_V, ti.BF16), q, ctxs[b],
                             w.rope_base)
        chk.close(got[b], ref, ti.BF16, f"seq {b}")
    chk.done()


@pytest.mark.parametrize("h,d_h,R_K,R_V,R_Q,ctx,chunk", [(32, 128, 4, 4, 6, 100, 64), (16, 64, 2, 2, 3, [37, 0], 300),
                                                          (32, 128, 4, 4, 6, [5, 130], 400),
                                                          (32, 128, 1, 1, 1, 0, 33), (20, 48, 1, 3, 16, 65, 40),
                                                          (64, 64, 1, 1, 4, [20, 3], 80), (16, 128, 2, 2, 5, 40, 300)])
def test_prefill_fq_matches_oracle(h, d_h, R_K, R_V, R_Q, ctx, chunk, request):
    """Causal chunk with factored query rows (row j at position ctx + j sees tokens 0 .. ctx + j)."""
    ctxs = ctx if isinstance(ctx, list) else [ctx]
    known = RANK1_PREFILL.get((h, d_h, R_K, R_V, R_Q, tuple(ctxs), chunk))
    if known:
        known_max_abs_excess(request, known, STORAGE_CAUSE)
    say(f"case: prefill fq h={h} d_h={d_h} R_K={R_K} R_V={R_V} R_Q={R_Q} ctx={ctxs} chunk={chunk}")
    _prefill_fq_case(h, d_h, R_K, R_V, R_Q, ctxs, chunk)


# Rank-1 factored-query prefill cases whose max-abs error exceeds 1e-2 (measured on MI355X; rel-L2 within 5e-3),
# keyed by (h, d_h, R_K, R_V, R_Q, ctx, chunk): a rank-1 query row of norm ~4 sharpens the softmax, and the
# bf16 values of the rotated B_K and of the built query row alone move the output that far.
RANK1_PREFILL = {(32, 128, 1, 1, 1, (0,), 33): "max-abs 1.772e-2, rel-L2 9.2e-4"}


@pytest.mark.parametrize("key", sorted(RANK1_PREFILL, key=str))
def test_prefill_fq_rank1_stored_values(key):
    """The listed cases against exact attention over the values the kernel reads: inside both plain bounds."""
    h, d_h, R_K, R_V, R_Q, ctxs, chunk = key
    say(f"case: prefill fq over stored values {key}")
    _prefill_fq_case(h, d_h, R_K, R_V, R_Q, list(ctxs), chunk, as_stored=True)
