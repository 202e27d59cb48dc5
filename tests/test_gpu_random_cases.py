"""Seeded random parity cases beyond the hand-picked ones: every compiled bf16 (heads, head dim) pair, ranks
1..4 (unequal R_K and R_V included), ragged and empty lengths, random split sizes and chunk geometry, all at
the plain bounds.  The softmax is left unsharpened (query scale 1 or 2): sharpened rank-1 cases sit on the
storage format's own floor and are covered, by name, in the other files."""
import numpy as np
import pytest

from tests.gpu_cases import (Checks, DecodeSetup, PrefillSetup, case_workload, random_sequences, say)

pytestmark = pytest.mark.gpu

SHAPES = [(16, 32), (16, 64), (16, 128), (32, 32), (32, 64), (32, 128), (64, 32), (64, 64)]


def padded_to(rng, h_pad: int, d_pad: int):
    """Random heads and (even) head dim that the library pads to (h_pad, d_pad): heads pad to a multiple of 16,
    a bf16 head dim to a multiple of 32; the full sizes half of the time."""
    if rng.integers(0, 2):
        return h_pad, d_pad
    return int(rng.integers(h_pad - 15, h_pad + 1)), 2 * int(rng.integers((d_pad - 32) // 2 + 1, d_pad // 2 + 1))


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    rng = np.random.default_rng(1000 + seed)
    h_pad, d_pad = SHAPES[seed % len(SHAPES)]
    h, d_h = padded_to(rng, h_pad, d_pad)
    R_K, R_V = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    batch = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 700, batch)]
    if seed % 3 == 0:
        lens[0] = 0
    q_scale = float(rng.choice([1.0, 2.0]))
    split = int(rng.choice([0, 0, 16, 64, 500]))
    w = case_workload(h, d_h, R_K, R_V)
    say(f"case: random decode seed {seed}: h={h} d_h={d_h} R_K={R_K} R_V={R_V} lens={lens} q_scale={q_scale} "
        f"split_tokens={split}")
    s = DecodeSetup(w, random_sequences(w, lens, q_scale=q_scale, seed=seed))
    ref = np.stack([s.oracle(b) for b in range(s.batch)])
    chk = Checks()
    chk.close(s.run(split_tokens=split), ref, w.dtype, f"split_tokens={split}")
    chk.done()


@pytest.mark.parametrize("seed", range(8))
def test_random_prefill(seed):
    rng = np.random.default_rng(2000 + seed)
    h_pad, d_pad = [(16, 64), (16, 128), (32, 64), (32, 128), (64, 64)][seed % 5]
    h, d_h = padded_to(rng, h_pad, d_pad)
    R_K, R_V = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    batch = int(rng.integers(1, 4))
    ctx = [int(x) for x in rng.integers(0, 400, batch)]
    chunk = int(rng.choice([1, 37, 256, 300, 513]))
    q_scale = float(rng.choice([1.0, 2.0]))
    w = case_workload(h, d_h, R_K, R_V)
    say(f"case: random prefill seed {seed}: h={h} d_h={d_h} R_K={R_K} R_V={R_V} ctx={ctx} chunk={chunk} "
        f"q_scale={q_scale}")
    seqs = random_sequences(w, [c + chunk for c in ctx], n_q=chunk, q_scale=q_scale, seed=seed)
    s = PrefillSetup(w, seqs, ctx)
    out = s.run()
    chk = Checks()
    for b in range(batch):
        chk.close(out[b], s.oracle(b), w.dtype, f"seq {b}")
    chk.done()
