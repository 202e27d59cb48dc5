"""GPU parity of tpa_prefill_chunk (causal chunk over a factor cache) against the fp64 oracle."""
import numpy as np
import pytest

import tpa_inputs as ti
from tests.gpu_cases import (DecodeSetup, PrefillSetup, assert_close, case_workload, random_sequences, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h,d_h,R", [(32, 128, 4), (32, 128, 1), (16, 64, 2), (20, 48, 3), (16, 128, 2), (64, 64, 1),
                                     (56, 64, 4)])
@pytest.mark.parametrize("ctx,chunk", [([0, 45, 300], 70), ([64, 2], 160), ([257], 129)])
@pytest.mark.parametrize("q_scale", [1.0, 10.0])
def test_small_chunks(h, d_h, R, ctx, chunk, q_scale):
    w = case_workload(h, d_h, R, R)
    say(f"case: prefill h={h} d_h={d_h} R={R} ctx={ctx} chunk={chunk} q_scale={q_scale}")
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, q_scale=q_scale, seed=h + chunk)
    s = PrefillSetup(w, seqs, ctx)
    out = s.run()
    ref = np.stack([s.oracle(b) for b in range(len(seqs))])
    assert_close(out, ref, w.dtype, "all rows")


def test_prefill_rows_match_gpu_decode():
    """Chunk row j equals a decode over the first ctx + j + 1 tokens with the query at position ctx + j."""
    w = case_workload(32, 128, 2, 2)
    ctx, chunk = 90, 40
    (seq,) = random_sequences(w, [ctx + chunk], n_q=chunk, q_scale=6.0, seed=21)
    pre = PrefillSetup(w, [seq], [ctx]).run()[0]
    rows = [0, 1, 17, 39]
    subs = [ti.Sequence(seq.A_K[:ctx + j + 1], seq.B_K[:ctx + j + 1], seq.A_V[:ctx + j + 1],
                        seq.B_V[:ctx + j + 1], seq.q[j:j + 1]) for j in rows]
    dec = DecodeSetup(w, subs, q_positions=[ctx + j for j in rows]).run()
    assert_close(pre[rows], dec, w.dtype, "prefill rows vs decodes")


def test_full_size_prefill_sampled_rows():
    """8 sequences x (2048 cached + 512-row causal chunk), h=32, d_h=128, R=4; oracle on sampled rows."""
    w = ti.get("c5")
    say(f"case: full-size prefill of {w.name}")
    seqs = ti.prefill_batch(w)
    s = PrefillSetup(w, seqs, [w.prefill_ctx] * w.prefill_batch)
    out = s.run()
    assert np.all(np.isfinite(out))
    rows = np.array([0, 1, 31, 32, 127, 128, 255, 256, 383, 384, 510, 511])
    for b in (0, 3, 7):
        assert_close(out[b][rows], s.oracle(b, rows=rows), w.dtype, f"seq {b} rows")


# Chunks of more than 256 rows at d_h = 128 run the wide form (512 query rows per work-group, factor
# pieces staged through LDS); these cases cover it with ragged chunk ends, a second row tile, short and
# empty contexts and every rank.
# (q_scale sets how peaked the softmax is: at R = 1 the rebuilt keys are largest, and a very peaked
# softmax over bf16 operands amplifies their rounding in the output, so the sharp case uses R = 4.)
@pytest.mark.parametrize("h,R,q_scale", [(32, 4, 2.0), (32, 2, 2.0), (32, 1, 2.0), (20, 4, 2.0), (16, 4, 2.0),
                                         (32, 4, 10.0)])
@pytest.mark.parametrize("ctx,chunk", [([0, 45], 300), ([257], 700), ([64, 1000, 3], 257)])
def test_wide_chunks(h, R, q_scale, ctx, chunk):
    w = case_workload(h, 128, R, R)
    say(f"case: wide prefill h={h} R={R} q_scale={q_scale} ctx={ctx} chunk={chunk}")
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, q_scale=q_scale, seed=h * R + chunk)
    s = PrefillSetup(w, seqs, ctx)
    out = s.run()
    ref = np.stack([s.oracle(b) for b in range(len(seqs))])
    assert_close(out, ref, w.dtype, "all rows")


@pytest.mark.parametrize("chunk", [100, 400])
def test_misaligned_start_gives_nan(chunk):
    """A sequence whose first slot is not a block boundary reports NaN rows; the others are unaffected."""
    w = case_workload(32, 128, 2, 2)
    say(f"case: misaligned prefill chunk={chunk}")
    ctx = [40, 70]
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, seed=chunk)
    s = PrefillSetup(w, seqs, ctx)
    bad = s.cache.seq_start.clone()
    bad[1] += 1
    out = s.run(seq_start=bad)
    assert np.all(np.isnan(out[1]))
    assert_close(out[0], s.oracle(0), w.dtype, "aligned sequence")


def test_wide_prefill_is_deterministic():
    w = case_workload(32, 128, 4, 4)
    seqs = random_sequences(w, [600, 333 + 300], n_q=300, seed=3)
    s = PrefillSetup(w, seqs, [300, 333])
    assert np.array_equal(s.run(), s.run())


@pytest.mark.parametrize("R_K,R_V", [(1, 3), (4, 2)])
def test_wide_unequal_ranks(R_K, R_V):
    """Unequal key and value ranks: the layout pads both to the larger rank with zero factor rows."""
    w = case_workload(32, 128, R_K, R_V)
    say(f"case: wide prefill R_K={R_K} R_V={R_V}")
    ctx, chunk = [33, 280], 290
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, q_scale=2.0, seed=R_K * 10 + R_V)
    s = PrefillSetup(w, seqs, ctx)
    out = s.run()
    ref = np.stack([s.oracle(b) for b in range(len(seqs))])
    assert_close(out, ref, w.dtype, "all rows")


@pytest.mark.parametrize("chunk", [120, 300])
def test_graph_replay_matches_eager(chunk):
    """Query RoPE (tpa_cache_append) + tpa_prefill_chunk recorded in a HIP graph (both prefill forms):
    every replay, with eager work in between, equals the eager result bit for bit."""
    import torch

    import factorized_kv_cache_tpa_amd as tpa
    from factorized_kv_cache_tpa_amd.cache import to_device
    w = case_workload(32, 128, 2, 2)
    say(f"case: prefill graph replay chunk={chunk}")
    ctx = [64, 200]
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, q_scale=2.0, seed=chunk + 5)
    s = PrefillSetup(w, seqs, ctx)
    eager = s.run()
    q = to_device(np.stack([x.q for x in seqs]), s.dims).reshape(len(seqs) * chunk, w.h, w.d_h)
    q_pos = torch.tensor(np.concatenate([c + np.arange(chunk) for c in ctx]), dtype=torch.int32, device="cuda")
    q_rot = torch.empty_like(q)
    out = torch.empty(len(seqs), chunk, w.h, w.d_h, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        s.cache.rotate_queries(q, q_pos, q_out=q_rot)
        tpa.tpa_prefill_chunk(s.dims, s.cache.buf, s.cache.capacity, s.cache.seq_start, s.ctx_len, max(ctx), chunk,
                              q_rot.view(len(seqs), chunk, w.h, w.d_h), out)
    for k in range(3):
        out.fill_(float("nan"))
        q_rot.zero_()
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {k}"
