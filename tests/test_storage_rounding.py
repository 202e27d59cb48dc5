"""The bf16 storage of rotated factors puts a floor under the error of any kernel that reads the cache.

The cache holds B_K rotated to each token's position and rounded to bf16 (RoPE is applied to the B factors
before they are stored: TPA notes page, RoPE compatibility), and tpa_decode takes the query rotated and
rounded the same way.  Exact attention over the values the cache and the query buffer hold therefore differs
from the oracle on the caller's unrotated factors, with no kernel involved.  For the sharpened rank-1 stress
inputs of the GPU parity tests this difference alone is above the 1e-2 max-abs bound, while rel-L2 stays well
inside 5e-3: those cases are listed as known max-abs excesses there.  Everything here runs on the CPU.
"""
import math

import numpy as np
import pytest

import oracle
import tpa_inputs as ti
from tests.gpu_cases import case_workload, random_sequences


def test_round_to_bf16_known_values_and_ties():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 unit at 1
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2.0 ** -40, -(one + ulp / 2),
                  3.0, 0.0, -0.0, 2.0 ** -126, 65504.0, 1e-30])
    got = oracle.round_to_bf16(x)
    want = [one, one, one + 2 * ulp, one + ulp, -one, 3.0, 0.0, -0.0, 2.0 ** -126, 65536.0, None]
    for g, w_, xi in zip(got, want, x):
        if w_ is not None:
            assert g == w_, (xi, g, w_)
    assert np.signbit(got[7])


def test_round_to_bf16_is_the_nearest_neighbour():
    """Brute force: the two bf16 values around x (from the fp32 bit pattern of a truncation) and an exact
    fp64 comparison of the distances, ties to the even pattern; 2e5 random magnitudes over 60 binades."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, 200_000))
    got = oracle.round_to_bf16(x)
    for xi, gi in zip(x[:5000], got[:5000]):
        m, e = math.frexp(abs(xi))  # xi = m 2^e, m in [0.5, 1)
        unit = 2.0 ** (e - 8)
        lo = math.floor(abs(xi) / unit) * unit
        hi = lo + unit
        dlo, dhi = abs(xi) - lo, hi - abs(xi)
        if dlo < dhi:
            r = lo
        elif dhi < dlo:
            r = hi
        else:
            r = lo if int(lo / unit) % 2 == 0 else hi
        assert gi == math.copysign(r, xi), (xi, gi, r)
    # on fp32-representable inputs it equals torch's bf16 cast (round to nearest even from fp32)
    torch = pytest.importorskip("torch")
    x32 = x.astype(np.float32)
    np.testing.assert_array_equal(oracle.round_to_bf16(x32.astype(np.float64)),
                                  torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy())


def _stored(x: np.ndarray, pos, base: float) -> np.ndarray:
    """What a bf16 buffer of x's rows rotated to pos holds (pos: per row, broadcast), rotated back exactly, so
    the oracle, which rotates whole rows itself, sees exactly the stored rotated values."""
    pos = np.asarray(pos, dtype=np.float64)
    return oracle.rope_rows_at(oracle.round_to_bf16(oracle.rope_rows_at(x, pos, base)), -pos, base)


@pytest.mark.parametrize("h,d_h", [(32, 128), (16, 64), (64, 64)])
def test_storage_floor_of_sharp_rank1_decode(h, d_h):
    """The decode stress inputs (rank 1, softmax sharpened 12x, lengths 1..600): exact attention over the
    stored values vs the oracle on the inputs."""
    w = case_workload(h, d_h, 1, 1)
    lens = [1, 7, 33, 100, 257, 600]
    seqs = random_sequences(w, lens, q_scale=12.0, seed=h * 31 + d_h)
    refs, stos = [], []
    for s, n in zip(seqs, lens):
        A_K, B_K, A_V, B_V, q = (ti.to_f64(x, w.dtype) for x in (s.A_K, s.B_K, s.A_V, s.B_V, s.q[:1]))
        refs.append(oracle.attention(A_K, B_K, A_V, B_V, np.arange(n), q, [n], [n], w.rope_base)[0])
        B_K_st = _stored(B_K, np.arange(n, dtype=np.float64)[:, None], w.rope_base)
        q_st = _stored(q, n, w.rope_base)
        stos.append(oracle.attention(A_K, B_K_st, A_V, B_V, np.arange(n), q_st, [n], [n], w.rope_base)[0])
    ref, sto = np.stack(refs), np.stack(stos)
    max_abs = float(np.abs(sto - ref).max())
    rel = float(np.linalg.norm(sto - ref) / np.linalg.norm(ref))
    print(f"h={h} d_h={d_h}: storage alone max_abs={max_abs:.3e} rel_l2={rel:.3e} max|out|={np.abs(ref).max():.2f}")
    assert max_abs > 1e-2 and rel < 5e-3


def test_storage_floor_is_small_on_the_measured_workloads():
    """The same floor on a sample of the 16 x 4096 workload (unsharpened query) is far inside both bounds."""
    w = ti.get("c2")
    for b in (0, 7):
        s = ti.decode_sequence(w, b)
        n = 512  # the first 512 tokens keep it quick; the query sits at position n
        A_K, B_K, A_V, B_V, q = (ti.to_f64(x[:n] if x is not s.q else x[:1], w.dtype)
                                 for x in (s.A_K, s.B_K, s.A_V, s.B_V, s.q))
        ref = oracle.attention(A_K, B_K, A_V, B_V, np.arange(n), q, [n], [n], w.rope_base)[0]
        B_K_st = _stored(B_K, np.arange(n, dtype=np.float64)[:, None], w.rope_base)
        sto = oracle.attention(A_K, B_K_st, A_V, B_V, np.arange(n), _stored(q, n, w.rope_base), [n], [n],
                               w.rope_base)[0]
        assert np.abs(sto - ref).max() < 1e-3
        assert np.linalg.norm(sto - ref) / np.linalg.norm(ref) < 1e-3
