"""GPU parity of the fused decode step, tpa_decode_step, against the fp64 oracle.

A step takes each sequence's N cached tokens plus the step's new token (unrotated factors)
and query (unrotated): the query at position N attends over all N + 1 tokens (the oracle's
causal row at position N, `oracle.prefill(..., ctx=N)`), and the new token's record lands
at slot N byte-for-byte as tpa_cache_append would write it.
"""
import numpy as np
import pytest
import torch

import factorized_kv_cache_tpa_amd as tpa
import oracle
import tpa_inputs as ti
from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device
from tests.gpu_cases import (STORAGE_CAUSE, Checks, assert_close, case_workload, dims_of, f64, known_max_abs_excess,
                             random_sequences, say, stored_factors, stored_key_and_query)

pytestmark = pytest.mark.gpu


class StepSetup:
    """N cached tokens per sequence (N = lens[b]) and the step's token N + query, all seeded."""

    def __init__(self, w: ti.Workload, lens, q_scale: float = 1.0, seed: int = 0, seqs=None, dims=None):
        self.w, self.dims, self.lens = w, dims_of(w) if dims is None else dims, list(lens)
        self.seqs = seqs if seqs is not None else random_sequences(w, [n + 1 for n in lens], q_scale=q_scale,
                                                                   seed=seed)
        self.cache = FactorCache(self.dims, [n + 1 for n in self.lens])
        for b, (s, n) in enumerate(zip(self.seqs, self.lens)):
            if n:
                self.cache.append_host(b, s.A_K[:n], s.B_K[:n], s.A_V[:n], s.B_V[:n])
        new = lambda x: to_device(np.stack([getattr(s, x)[n] for s, n in zip(self.seqs, self.lens)]), self.dims)
        self.A_K, self.B_K, self.A_V, self.B_V = (new(x) for x in ("A_K", "B_K", "A_V", "B_V"))
        self.q = to_device(np.stack([s.q[0] for s in self.seqs]), self.dims)
        self.seq_len = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.batch, self.max_len = len(self.lens), max(self.lens)

    def workspace(self, split_tokens: int = 0) -> torch.Tensor:
        n = tpa.tpa_decode_workspace_bytes(self.dims, self.batch, self.max_len, split_tokens)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")

    def run(self, split_tokens: int = 0, seq_start=None, out=None, ws=None, capacity=None) -> torch.Tensor:
        """capacity: the capacity the call declares (default the cache's own)."""
        out = torch.full((self.batch, self.w.h, self.w.d_h), float("nan"), dtype=torch.float32,
                         device="cuda") if out is None else out
        ws = self.workspace(split_tokens) if ws is None else ws
        tpa.tpa_decode_step(self.dims, self.cache.buf, self.cache.capacity if capacity is None else capacity,
                            self.cache.seq_start if seq_start is None else seq_start, self.seq_len, self.max_len,
                            self.A_K, self.B_K, self.A_V, self.B_V, self.q, out, ws, split_tokens=split_tokens)
        return out

    def oracle(self, b: int, as_stored: bool = False) -> np.ndarray:
        """as_stored: over the values the kernel reads (B_K rotated and rounded to bf16 per token, the new
        token's included, and the query rotated to position N and rounded) instead of the caller's factors."""
        s, n, dt = self.seqs[b], self.lens[b], self.w.dtype
        A_K, B_K, A_V, B_V = stored_factors(s, n + 1, self.w, self.dims)
        q = f64(s.q[:1], dt)
        if as_stored:
            B_K, q = stored_key_and_query(B_K, q, [n], self.w, self.dims)
        return oracle.prefill(A_K, B_K, A_V, B_V, q, n, self.w.rope_base)[0]


SHAPES = [(32, 128, 1, 1, ti.BF16, 1e4), (16, 64, 2, 2, ti.BF16, 1e4), (32, 128, 4, 4, ti.BF16, 5e5),
          (20, 48, 1, 3, ti.BF16, 1e4), (4, 16, 1, 1, ti.F32, 1e4), (32, 128, 3, 2, ti.F32, 5e5),
          (64, 64, 1, 1, ti.BF16, 1e4), (56, 32, 2, 2, ti.BF16, 1e4), (16, 128, 2, 2, ti.BF16, 5e5),
          (30, 64, 2, 1, ti.F32, 1e4)]


STEP_LENS = [0, 1, 31, 32, 33, 300, 1000]
# Sharpened rank-1 cases whose max-abs error exceeds 1e-2 (measured on MI355X; rel-L2 within 5e-3), keyed by
# (h, d_h, R_K, R_V, dtype, base, q_scale).  Exact attention over the stored rotated B_K and query, on the
# CPU, is 1.035e-2 away from the oracle for the sequence of N = 31 alone.
SHARP_RANK1 = {(64, 64, 1, 1, ti.BF16, 1e4, 6.0): "max-abs 1.006e-2 (N = 31), rel-L2 2.6e-3"}


@pytest.mark.parametrize("h,d_h,R_K,R_V,dtype,base", SHAPES)
@pytest.mark.parametrize("q_scale", [1.0, 6.0])
def test_step_matches_oracle(h, d_h, R_K, R_V, dtype, base, q_scale, request):
    known = SHARP_RANK1.get((h, d_h, R_K, R_V, dtype, base, q_scale))
    if known:
        known_max_abs_excess(request, known, STORAGE_CAUSE)
    w = case_workload(h, d_h, R_K, R_V, dtype, base)
    say(f"case: step h={h} d_h={d_h} R_K={R_K} R_V={R_V} {dtype} q_scale={q_scale} lens={STEP_LENS}")
    st = StepSetup(w, STEP_LENS, q_scale=q_scale, seed=h + d_h + R_K)
    got = st.run().cpu().numpy()
    chk = Checks()
    for b in range(st.batch):
        chk.close(got[b], st.oracle(b), dtype, f"seq {b} (N={STEP_LENS[b]})")
    chk.done()


@pytest.mark.parametrize("key", sorted(SHARP_RANK1, key=str))
def test_step_sharp_rank1_stored_values(key):
    """The listed cases against exact attention over the values the kernel reads: inside both plain bounds."""
    h, d_h, R_K, R_V, dtype, base, q_scale = key
    w = case_workload(h, d_h, R_K, R_V, dtype, base)
    say(f"case: step over stored values {key}")
    st = StepSetup(w, STEP_LENS, q_scale=q_scale, seed=h + d_h + R_K)
    got = st.run().cpu().numpy()
    chk = Checks()
    for b in range(st.batch):
        chk.close(got[b], st.oracle(b, as_stored=True), dtype, f"seq {b} (N={STEP_LENS[b]})")
    chk.done()


def test_step_with_no_cached_tokens_returns_the_new_value_row():
    """N = 0: the query sees only the new token, so out = V_new = (1/R_V) A_V^T B_V."""
    w = case_workload(32, 128, 2, 2, ti.BF16)
    st = StepSetup(w, [0, 0], seed=3)
    got = st.run().cpu().numpy()
    for b in range(2):
        s = st.seqs[b]
        v = f64(s.A_V[0], ti.BF16).T @ f64(s.B_V[0], ti.BF16) / 2.0
        assert_close(got[b], v, ti.BF16, f"seq {b}")


def check_record_is_what_append_writes(st: StepSetup, lens):
    st.run()
    # the same tokens through tpa_cache_append into a fresh cache of the same geometry
    ref = FactorCache(st.dims, [n + 1 for n in lens])
    slots = torch.tensor([ref.starts[b] + n for b, n in enumerate(lens)], dtype=torch.int64, device="cuda")
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tpa.tpa_cache_append(st.dims, ref.buf, ref.capacity, slots, pos, st.A_K, st.B_K, st.A_V, st.B_V)
    reads = []
    for cache in (st.cache, ref):
        outs = [torch.zeros(x.shape, dtype=st.dims.cache_torch_dtype, device="cuda")
                for x in (st.A_K, st.B_K, st.A_V, st.B_V)]
        tpa.tpa_cache_read(st.dims, cache.buf, cache.capacity, slots, *outs)
        reads.append(outs)
    torch.cuda.synchronize()
    for name, a, b in zip(("A_K", "B_K", "A_V", "B_V"), *reads):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


@pytest.mark.parametrize("h,d_h,R_K,R_V,dtype,base", SHAPES)
def test_step_record_is_what_append_writes(h, d_h, R_K, R_V, dtype, base):
    w = case_workload(h, d_h, R_K, R_V, dtype, base)
    lens = [5, 40, 131]
    check_record_is_what_append_writes(StepSetup(w, lens, seed=11), lens)


def test_decode_after_step_sees_the_written_token():
    """A plain decode over N + 1 tokens (the record the step wrote) with the query rotated at N."""
    w = case_workload(32, 128, 1, 1, ti.BF16)
    lens = [7, 64, 129]
    st = StepSetup(w, lens, seed=5)
    st.run()
    q_rot = st.cache.rotate_queries(st.q, st.seq_len)
    ws = torch.zeros(tpa.tpa_decode_workspace_bytes(st.dims, st.batch, st.max_len + 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(st.batch, w.h, w.d_h, dtype=torch.float32, device="cuda")
    tpa.tpa_decode(st.dims, st.cache.buf, st.cache.capacity, st.cache.seq_start, st.seq_len + 1, st.max_len + 1,
                   q_rot, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(st.batch):
        assert_close(got[b], st.oracle(b), ti.BF16, f"seq {b}")


@pytest.mark.parametrize("split_tokens", [32, 96, 256, 4096])
def test_step_split_sizes(split_tokens):
    w = case_workload(32, 128, 2, 2, ti.BF16)
    lens = [1, 100, 777, 2000]
    st = StepSetup(w, lens, q_scale=6.0, seed=21)
    got = st.run(split_tokens=split_tokens).cpu().numpy()
    for b in range(st.batch):
        assert_close(got[b], st.oracle(b), ti.BF16, f"split {split_tokens} seq {b}")


def test_step_full_size_decode_b16_h32_d128_r1_n4096():
    """The metric's workload: 16 sequences of 4096 cached tokens, every sequence checked."""
    w = ti.get("rank1")
    say(f"case: step full size {w.name}")
    lens = list(ti.decode_lengths(w))
    seqs = []
    for b in range(w.batch):  # one more token than the workload's cache: the step's new token
        seqs.append(ti.draw_sequence(np.random.SeedSequence([w.seed, 77, b]), lens[b] + 1, 1, w))
    st = StepSetup(w, lens, seqs=seqs)
    got = st.run().cpu().numpy()
    for b in range(st.batch):
        assert_close(got[b], st.oracle(b), w.dtype, f"seq {b}")


def test_step_misaligned_start_gives_nan_and_writes_nothing():
    w = case_workload(32, 128, 1, 1, ti.BF16)
    st = StepSetup(w, [40, 40], seed=9)
    before = st.cache.buf.clone()
    bad = st.cache.seq_start.clone()
    bad[1] += 1  # not a block boundary
    got = st.run(seq_start=bad).cpu().numpy()
    assert np.all(np.isnan(got[1]))
    assert_close(got[0], st.oracle(0), ti.BF16, "seq 0")
    # only sequence 0's slot 40 changed
    changed = (st.cache.buf != before).nonzero().flatten()
    blk = tpa.tpa_cache_bytes(st.dims, tpa.tpa_block_tokens(st.dims))
    assert changed.numel() > 0
    assert int(changed.min()) >= (40 // 32) * blk and int(changed.max()) < (40 // 32 + 1) * blk


def test_step_new_slot_past_capacity_gives_nan_and_writes_nothing():
    """The cached tokens fit the declared capacity but the new token's slot does not: NaN output for that
    sequence and no write; the other sequence steps normally.  The buffer holds more than the declared
    capacity, so a missed guard would write inside the allocation (and be seen), never fault."""
    w = case_workload(32, 128, 1, 1, ti.BF16)
    lens = [40, 70]
    st = StepSetup(w, lens, seed=19)
    declared = st.cache.starts[1] + lens[1]  # sequence 1's slot 70 is the first slot past it
    before = st.cache.buf.clone()
    got = st.run(capacity=declared).cpu().numpy()
    assert np.all(np.isnan(got[1]))
    assert_close(got[0], st.oracle(0), ti.BF16, "seq 0")
    changed = (st.cache.buf != before).nonzero().flatten()
    blk = tpa.tpa_cache_bytes(st.dims, tpa.tpa_block_tokens(st.dims))
    assert changed.numel() > 0
    assert int(changed.min()) >= (40 // 32) * blk and int(changed.max()) < (40 // 32 + 1) * blk


def test_step_graph_replays_match_eager():
    """Captured once, replayed several times with eager work in between: each replay reproduces the
    eager output bit for bit (the step is deterministic and rewrites the same record)."""
    w = case_workload(32, 128, 1, 1, ti.BF16)
    st = StepSetup(w, [100, 2048, 4000], seed=13)
    ws = st.workspace()
    eager = st.run(ws=ws).clone()
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        st.run(out=out, ws=ws)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del junk


def test_step_over_more_than_256_sequences():
    """A fused step over 400 short ragged sequences (empty ones included): every output and every written
    record against the oracle and the append."""
    w = case_workload(32, 128, 1, 1, ti.BF16, 1e4)
    lens = [int(x) for x in np.random.default_rng(11).integers(0, 40, 400)]
    say(f"case: step over {len(lens)} sequences")
    st = StepSetup(w, lens, seed=400)
    got = st.run().cpu().numpy()
    chk = Checks()
    for b in range(st.batch):
        chk.close(got[b], st.oracle(b), w.dtype, f"seq {b} (N={lens[b]})")
    chk.done()
    check_record_is_what_append_writes(st, lens)
