"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print, a closed form derived by hand, a textbook library routine
(torch scaled_dot_product_attention in fp64), an independent brute force, or
an invariant that a dropped term, a wrong sign, a wrong pairing or a
transposed operand would break.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import tpa_inputs as ti
from tests import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, n, h, d, RK, RV, n_q=1, q_scale=1.0):
    s = ti.random_case(seed, n, n_q, h, d, RK, RV, ti.F32, q_scale)
    f = lambda a: ti.to_f64(a, ti.F32)
    return f(s.A_K), f(s.B_K), f(s.A_V), f(s.B_V), f(s.q)


# --- cache size: the page's worked example --------------------------------------------------------

def test_cache_size_matches_page_example():
    g = json.load(open(os.path.join(GOLDEN, "cache_size_page.json")))
    assert oracle.factor_elems_per_token(g["h"], g["d_h"], g["R_K"], g["R_V"]) == g["tpa_elements_per_token"]
    assert oracle.dense_elems_per_token(g["h"], g["d_h"]) == g["mha_elements_per_token"]


@pytest.mark.parametrize("h,d,R,tpa,dense", [(16, 64, 2, 320, 2048), (32, 128, 2, 640, 8192),
                                             (32, 128, 4, 1280, 8192), (4, 16, 1, 40, 128)])
def test_cache_size_other_shapes(h, d, R, tpa, dense):
    assert oracle.factor_elems_per_token(h, d, R, R) == tpa
    assert oracle.dense_elems_per_token(h, d) == dense


# --- RoPE: convention pinned by the complex form and by Theorem 3.1 --------------------------------

@pytest.mark.parametrize("d,pos,base", [(2, 3, 1e4), (16, 64, 1e4), (128, 4096, 1e4), (128, 131071, 5e5),
                                        (64, 0, 1e4)])
def test_rope_equals_complex_rotation(d, pos, base):
    x = np.random.default_rng(d + pos).standard_normal((3, d))
    got = oracle.rope_rows(x, pos, base)
    j = np.arange(d // 2)
    theta = np.power(base, -2.0 * j / d)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos * theta)
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = z.real, z.imag
    # the angle p * theta_j carries an fp64 rounding error of about p * 2^-52 (libm pow vs numpy power),
    # so the bound grows with the position
    np.testing.assert_allclose(got, want, rtol=0, atol=4e-16 * (pos + 16) * np.abs(x).max())


def _rot_matrix(d, angle_mult, base):
    """Block-diagonal rotation acting on column vectors: pair j turns by angle_mult * theta_j."""
    T = np.zeros((d, d))
    for j in range(d // 2):
        a = angle_mult * base ** (-2.0 * j / d)
        c, s = math.cos(a), math.sin(a)
        T[2 * j:2 * j + 2, 2 * j:2 * j + 2] = [[c, -s], [s, c]]
    return T


def test_rope_relative_position_theorem():
    """Scores from rotated q and rotated K equal q T_{t-s} K^T built from the unrotated rows."""
    rng = np.random.default_rng(7)
    d, base = 16, 1e4
    for t, s in [(5, 2), (64, 0), (100, 99), (4096, 17)]:
        q = rng.standard_normal(d)
        k = rng.standard_normal(d)
        lhs = float(oracle.rope_rows(q, t, base) @ oracle.rope_rows(k, s, base))
        # q~ . k~ = q^T R_t^T R_s k, and R_t^T R_s is the block rotation by (s - t)
        T = _rot_matrix(d, s - t, base)
        rhs = float(q @ T @ k)
        assert abs(lhs - rhs) < 1e-12 * (1 + abs(rhs))
        # depends on t - s only
        T2 = _rot_matrix(d, (s + 37) - (t + 37), base)
        assert np.allclose(T, T2, atol=1e-12)


def test_attention_matches_theorem_form_two_tokens():
    """Full oracle output equals softmax over q T_{t-s} K_s^T (unrotated K_s from the factors)."""
    A_K, B_K, A_V, B_V, q = _rand(11, 5, 3, 8, 2, 3)
    base, t = 1e4, 9
    pos = np.array([0, 3, 4, 7, 8])
    got = oracle.attention(A_K, B_K, A_V, B_V, pos, q, [t], [5], base)[0]
    for i in range(3):
        z, vals = [], []
        for s in range(5):
            k = sum(np.outer(A_K[s, r], B_K[s, r]) for r in range(2))[i] / 2
            v = sum(np.outer(A_V[s, r], B_V[s, r]) for r in range(3))[i] / 3
            z.append(q[0, i] @ _rot_matrix(8, pos[s] - t, base) @ k / math.sqrt(8))
            vals.append(v)
        w = np.exp(np.array(z) - max(z))
        w /= w.sum()
        np.testing.assert_allclose(got[i], w @ np.array(vals), rtol=0, atol=1e-12)


def test_shift_of_all_positions_leaves_output_unchanged():
    A_K, B_K, A_V, B_V, q = _rand(12, 9, 4, 16, 2, 2, q_scale=4.0)
    pos = np.arange(9)
    a = oracle.attention(A_K, B_K, A_V, B_V, pos, q, [9], [9], 1e4)
    b = oracle.attention(A_K, B_K, A_V, B_V, pos + 1000, q, [1009], [9], 1e4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


def test_closed_form_two_tokens():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_two_tokens.json")))
    inp = g["inputs"]
    got = oracle.attention(inp["A_K"], inp["B_K"], inp["A_V"], inp["B_V"], inp["kv_positions"], [inp["q"]],
                           [inp["q_position"]], [2], inp["rope_base"])[0, 0]
    z0, z1 = math.cos(2) / math.sqrt(2), math.sin(1) / math.sqrt(2)
    e0, e1 = math.exp(z0), math.exp(z1)
    w0, w1 = e0 / (e0 + e1), e1 / (e0 + e1)
    np.testing.assert_allclose(got, [w0 + 3 * w1, 2 * w0 + 4 * w1], rtol=0, atol=1e-14)


# --- reduction to textbook multi-head attention -----------------------------------------------------

def _sdpa(q_rot, K_rot, V, scale):
    """torch's textbook scaled dot-product attention, fp64 on the CPU. q [h][d], K/V [n][h][d]."""
    qt = torch.from_numpy(q_rot)[:, None, :]           # [h][1][d]
    kt = torch.from_numpy(np.ascontiguousarray(K_rot.transpose(1, 0, 2)))  # [h][n][d]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("h,d,n", [(4, 16, 64), (3, 8, 7), (8, 32, 33)])
def test_reduces_to_mha_with_permutation_head_factors(h, d, n):
    """R = h and A = R * P (P a non-involutive permutation): K_s rows are B_K rows permuted.

    K_s[i,:] = (1/R) sum_r A[r][i] B[r,:] = B[perm(i),:].  A transposed head factor would pick
    B[perm^-1(i),:] instead, and a dropped 1/R would scale K and V by R; both fail here.
    """
    rng = np.random.default_rng(h * 100 + n)
    R = h
    perm = np.roll(np.arange(h), 1)  # i -> i-1 (mod h), not its own inverse for h > 2
    A = np.zeros((R, h))
    A[perm, np.arange(h)] = R
    B_K = rng.standard_normal((n, R, d))
    B_V = rng.standard_normal((n, R, d))
    q = rng.standard_normal((h, d))
    A_b = np.broadcast_to(A, (n, R, h))
    base = 1e4
    got = oracle.decode(A_b, B_K, A_b, B_V, q, base)
    K = B_K[:, perm, :]
    V = B_V[:, perm, :]
    # RoPE applied with the complex form of the brute force (pinned above), not the oracle's own
    K_rot = np.array([[brute_force.rope_complex(list(K[s, i]), s, base) for i in range(h)] for s in range(n)])
    q_rot = np.array([brute_force.rope_complex(list(q[i]), n, base) for i in range(h)])
    want = _sdpa(q_rot, K_rot, V, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# --- special cases and invariants ---------------------------------------------------------------------

@pytest.mark.parametrize("R", [1, 2, 4])
def test_single_cached_token_returns_its_value(R):
    A_K, B_K, A_V, B_V, q = _rand(20 + R, 1, 4, 16, R, R, q_scale=3.0)
    got = oracle.decode(A_K, B_K, A_V, B_V, q[0], 1e4)
    want = sum(np.outer(A_V[0, r], B_V[0, r]) for r in range(R)) / R
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_zero_query_averages_values():
    A_K, B_K, A_V, B_V, q = _rand(30, 17, 4, 16, 2, 3)
    got = oracle.decode(A_K, B_K, A_V, B_V, np.zeros_like(q[0]), 1e4)
    V = np.einsum("srh,srd->shd", A_V, B_V) / 3
    np.testing.assert_allclose(got, V.mean(axis=0), rtol=0, atol=1e-14)


def test_factor_rescaling_and_rank_permutation_invariance():
    A_K, B_K, A_V, B_V, q = _rand(31, 23, 4, 16, 3, 2, q_scale=5.0)
    ref = oracle.decode(A_K, B_K, A_V, B_V, q[0], 1e4)
    c = np.array([2.0, -0.5, 4.0])[None, :, None]
    cv = np.array([0.25, -3.0])[None, :, None]
    got = oracle.decode(A_K * c, B_K / c, A_V * cv, B_V / cv, q[0], 1e4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    pk, pv = [2, 0, 1], [1, 0]
    got = oracle.decode(A_K[:, pk], B_K[:, pk], A_V[:, pv], B_V[:, pv], q[0], 1e4)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_outputs_lie_in_convex_hull_of_values():
    A_K, B_K, A_V, B_V, q = _rand(32, 40, 4, 16, 2, 2, q_scale=8.0)
    got = oracle.decode(A_K, B_K, A_V, B_V, q[0], 1e4)
    V = np.einsum("srh,srd->shd", A_V, B_V) / 2
    assert np.all(got <= V.max(axis=0) + 1e-12) and np.all(got >= V.min(axis=0) - 1e-12)


def test_no_visible_tokens_gives_zeros():
    A_K, B_K, A_V, B_V, q = _rand(33, 4, 2, 8, 1, 1)
    got = oracle.attention(A_K, B_K, A_V, B_V, np.arange(4), q, [4], [0], 1e4)
    assert np.all(got == 0.0)


def test_prefill_rows_equal_decodes():
    s = ti.random_case(40, 12, 5, 4, 16, 2, 2, ti.F32, q_scale=4.0)
    f = lambda a: ti.to_f64(a, ti.F32)
    A_K, B_K, A_V, B_V, q = map(f, (s.A_K, s.B_K, s.A_V, s.B_V, s.q))
    ctx = 7
    pre = oracle.prefill(A_K, B_K, A_V, B_V, q, ctx, 1e4)
    for j in range(5):
        n = ctx + j + 1
        dec = oracle.attention(A_K[:n], B_K[:n], A_V[:n], B_V[:n], np.arange(n), q[j:j + 1], [ctx + j], [n], 1e4)
        np.testing.assert_allclose(pre[j], dec[0], rtol=0, atol=1e-14)


# --- brute force on tiny random shapes ---------------------------------------------------------------

@pytest.mark.parametrize("h,d,RK,RV,n", [(1, 2, 1, 1, 1), (2, 4, 2, 1, 2), (4, 16, 1, 1, 64), (2, 16, 3, 2, 7),
                                         (4, 4, 2, 3, 5)])
def test_brute_force_agreement(h, d, RK, RV, n):
    A_K, B_K, A_V, B_V, q = _rand(50 + n, n, h, d, RK, RV, n_q=2, q_scale=4.0)
    pos = np.arange(n)
    q_pos, q_nvis = [n, n - 1], [n, max(0, n - 1)]
    got = oracle.attention(A_K, B_K, A_V, B_V, pos, q, q_pos, q_nvis, 1e4)
    want = brute_force.attention(A_K.tolist(), B_K.tolist(), A_V.tolist(), B_V.tolist(), pos.tolist(),
                                 q.tolist(), q_pos, q_nvis, 1e4)
    np.testing.assert_allclose(got, np.array(want), rtol=0, atol=1e-12)


def test_brute_force_on_tiny_fp32_workload():
    """The tiny fp32 decode workload itself (h=4, d_h=16, R=1, 64 cached tokens, query at 64)."""
    w = ti.get("tiny")
    s = ti.decode_sequence(w, 0)
    f = lambda a: ti.to_f64(a, w.dtype)
    A_K, B_K, A_V, B_V, q = map(f, (s.A_K, s.B_K, s.A_V, s.B_V, s.q))
    got = oracle.decode(A_K, B_K, A_V, B_V, q[0], w.rope_base)
    want = brute_force.attention(A_K.tolist(), B_K.tolist(), A_V.tolist(), B_V.tolist(), list(range(64)),
                                 q.tolist(), [64], [64], w.rope_base)
    np.testing.assert_allclose(got, np.array(want)[0], rtol=0, atol=1e-12)


# --- factored query (full TPA: Q = (1/R_Q) A_Q^T B_Q, same tensor product decomposition) --------------

def test_query_factors_with_permutation_head_factor_select_rows():
    """R_Q = h and A_Q = R_Q * P (P a permutation with no fixed points): q[i] is exactly row P(i) of B_Q,
    so a transposed head factor, a dropped 1/R_Q or a wrong index fails."""
    h, d = 5, 6
    perm = [2, 3, 4, 0, 1]
    rng = np.random.default_rng(3)
    B_Q = rng.standard_normal((1, h, d))
    A_Q = np.zeros((1, h, h))
    for i in range(h):
        A_Q[0, perm[i], i] = h
    q = oracle.query_from_factors(A_Q, B_Q)[0]
    for i in range(h):  # (h * x) / h is x to within one rounding
        np.testing.assert_allclose(q[i], B_Q[0, perm[i]], rtol=2.3e-16, atol=0)


@pytest.mark.parametrize("h,d,RQ", [(1, 2, 1), (4, 16, 3), (3, 8, 6)])
def test_query_factors_match_brute_force(h, d, RQ):
    rng = np.random.default_rng(h * 10 + RQ)
    A_Q, B_Q = rng.standard_normal((2, RQ, h)), rng.standard_normal((2, RQ, d))
    got = oracle.query_from_factors(A_Q, B_Q)
    for t in range(2):
        want = brute_force.query_from_factors(A_Q[t].tolist(), B_Q[t].tolist())
        np.testing.assert_allclose(got[t], np.array(want), rtol=0, atol=1e-14)


def test_query_factor_rank_permutation_and_rescaling_invariance():
    rng = np.random.default_rng(8)
    A_Q, B_Q = rng.standard_normal((1, 4, 6)), rng.standard_normal((1, 4, 10))
    q = oracle.query_from_factors(A_Q, B_Q)
    perm = [3, 1, 0, 2]
    np.testing.assert_allclose(oracle.query_from_factors(A_Q[:, perm], B_Q[:, perm]), q, rtol=0, atol=1e-14)
    c = np.array([2.0, -0.5, 4.0, 0.25])[None, :, None]
    np.testing.assert_allclose(oracle.query_from_factors(A_Q * c, B_Q / c), q, rtol=0, atol=1e-13)


def test_rope_of_query_factors_commutes_with_their_combination():
    """Rotating the B_Q rows at a position and then combining equals combining and then rotating (RoPE is
    linear), which is why the feature factor alone can be rotated (RoPE compatibility, Theorem 3.1)."""
    rng = np.random.default_rng(9)
    A_Q, B_Q = rng.standard_normal((1, 3, 4)), rng.standard_normal((1, 3, 16))
    for pos in (0, 7, 4096, 131071):
        a = oracle.rope_rows(oracle.query_from_factors(A_Q, B_Q)[0], pos, 1e4)
        b = oracle.query_from_factors(A_Q, oracle.rope_rows(B_Q[0], pos, 1e4)[None])[0]
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_factored_query_decode_matches_brute_force():
    """Full pipeline on a tiny case: query built from factors, then decode, against the brute force's own
    query combination and attention."""
    h, d, RK, RV, RQ, n = 4, 8, 2, 2, 3, 9
    A_K, B_K, A_V, B_V, _ = _rand(77, n, h, d, RK, RV)
    rng = np.random.default_rng(77)
    A_Q, B_Q = rng.standard_normal((1, RQ, h)), rng.standard_normal((1, RQ, d))
    q = oracle.query_from_factors(A_Q, B_Q)
    got = oracle.decode(A_K, B_K, A_V, B_V, q[0], 1e4)
    qb = brute_force.query_from_factors(A_Q[0].tolist(), B_Q[0].tolist())
    want = brute_force.attention(A_K.tolist(), B_K.tolist(), A_V.tolist(), B_V.tolist(), list(range(n)), [qb],
                                 [n], [n], 1e4)
    np.testing.assert_allclose(got, np.array(want)[0], rtol=0, atol=1e-12)


# ---- OCP E4M3 codec used for 8-bit factor storage (OCP 8-bit floating point specification, E4M3)

def test_e4m3_known_codes():
    """Values fixed by the format: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448,
    S.1111.111 is NaN, sign bit 7."""
    v = oracle.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x30, 0x38, 0x3C, 0x40, 0x77, 0x7E, 0x7F,
                                     0x80, 0x81, 0xB8, 0xFE, 0xFF], dtype=np.uint8))
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 0.5, 1.0, 1.5, 2.0, 240.0, 448.0, np.nan,
            -0.0, -(2.0 ** -9), -1.0, -448.0, np.nan]
    np.testing.assert_array_equal(v, want)
    assert math.copysign(1.0, v[11]) == -1.0  # 0x80 is negative zero


def test_e4m3_finite_codes_are_monotone_and_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(codes)
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)  # 0x00 .. 0x7E strictly increasing
    np.testing.assert_array_equal(v[128:255], -pos)  # sign bit mirrors
    finite = np.isfinite(v)
    assert finite.sum() == 254
    np.testing.assert_array_equal(oracle.e4m3_encode(v[finite]), codes[finite])


def test_e4m3_ties_go_to_even_and_range_ends():
    v = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2  # exact in fp64
    got = oracle.e4m3_encode(mids)
    lower = np.arange(126)
    np.testing.assert_array_equal(got, np.where(lower % 2 == 0, lower, lower + 1))
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, np.inf)), lower + 1)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, -np.inf)), lower)
    # saturation past 448 (no infinities in E4M3), signed underflow, NaN
    np.testing.assert_array_equal(oracle.e4m3_encode([449.0, 464.0, 1e30, -1e30, np.inf, -np.inf]),
                                  [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE])
    np.testing.assert_array_equal(oracle.e4m3_encode([2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, 1.5 * 2.0 ** -10]),
                                  [0x00, 0x80, 0x00, 0x01])
    assert oracle.e4m3_encode([np.nan])[0] == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    """torch's float8_e4m3fn cast (an independent implementation of the same format, round to nearest
    even) agrees on every in-range value."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-9.0, 6.0, 200000))
    x = x[np.abs(x) <= 448.0]
    want = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), want)
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_decode(codes), tv)


def test_rope_rows_at_equals_row_by_row_rotation():
    """The batched rotation is the per-row rotation, row for row, at each row's own position."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 3, 16))
    pos = rng.integers(0, 100000, size=(7, 1)).astype(np.float64)
    got = oracle.rope_rows_at(x, pos, 500000.0)
    for t in range(7):
        np.testing.assert_array_equal(got[t], oracle.rope_rows(x[t], float(pos[t, 0]), 500000.0))


@pytest.mark.parametrize("cuts", [[0, 40], [0, 1, 40], [0, 13, 14, 29, 40], list(range(0, 41, 5)),
                                  [0, 39, 40], "random"])
def test_split_merge_algebra_equals_one_pass(cuts):
    """Pin O7: cut the cached tokens into contiguous pieces; per piece j and head, m_j = max score, l_j = sum of
    exp(score - m_j) (scores from the independent brute force) and O_j = the piece's normalized attention
    output (the oracle over that piece alone, tokens at their own positions).  The textbook merge
    M = max m_j, out = sum_j e^(m_j - M) l_j O_j / sum_j e^(m_j - M) l_j must give the one-pass output: the rule
    the split-sequence decode applies to its partials.  Sharpened query, so the pieces' masses differ widely."""
    rng = np.random.default_rng(707)
    h, d, RK, RV, N, base = 3, 8, 2, 3, 40, 1e4
    A_K = rng.standard_normal((N, RK, h)) / np.sqrt(RK)
    B_K = rng.standard_normal((N, RK, d)) / np.sqrt(RK)
    A_V = rng.standard_normal((N, RV, h)) / np.sqrt(RV)
    B_V = rng.standard_normal((N, RV, d)) / np.sqrt(RV)
    q = 4.0 * rng.standard_normal((h, d))
    if cuts == "random":
        cuts = [0] + sorted(int(c) for c in rng.choice(np.arange(1, N), 6, replace=False)) + [N]
    full = oracle.decode(A_K, B_K, A_V, B_V, q, base)
    z_all = [brute_force.scores(A_K.tolist(), B_K.tolist(), list(range(N)), q[i].tolist(), N, i, base)
             for i in range(h)]
    pieces = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        O = oracle.attention(A_K[a:b], B_K[a:b], A_V[a:b], B_V[a:b], np.arange(a, b), q[None], [N], [b - a],
                             base)[0]
        ml = []
        for i in range(h):
            z = z_all[i][a:b]
            m = max(z)
            ml.append((m, math.fsum(math.exp(x - m) for x in z)))
        pieces.append((ml, O))
    for i in range(h):
        M = max(ml[i][0] for ml, _ in pieces)
        w = [math.exp(ml[i][0] - M) * ml[i][1] for ml, _ in pieces]
        merged = sum(wj * O[i] for wj, (_, O) in zip(w, pieces)) / math.fsum(w)
        np.testing.assert_allclose(merged, full[i], rtol=0, atol=1e-12)
    if len(cuts) > 2:  # a wrong rule (the pieces' outputs averaged, masses ignored) is far off
        avg = np.mean([O for _, O in pieces], axis=0)
        assert np.abs(avg - full).max() > 1e-3


@pytest.mark.parametrize("d,pos,base", [(8, 3.0, 1e4), (16, 1000.0, 1e4), (128, 131071.0, 5e5)])
def test_half_split_rotation_is_a_channel_permutation_of_the_pair_rotation(d, pos, base):
    """Pin O2b (reading R2: pairs (2j, 2j+1)).  The half-split convention rotates (x_j, x_{j+d/2}) by the same
    angle pos * base^(-2j/d); with P the permutation taking channel 2j to j and 2j+1 to j + d/2, the half-split
    rotation of P x equals P times the oracle's rotation of x.  The oracle does not itself equal the half-split
    form, so the convention is fixed, and a half-split caller permutes its channels once."""
    rng = np.random.default_rng(int(d + pos) % 2**32)
    x = rng.standard_normal((5, d))
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # (P x)[k] = x[perm[k]]
    half = d // 2
    ang = pos * base ** (-2.0 * np.arange(half) / d)
    c, s = np.cos(ang), np.sin(ang)

    def half_split(v):
        a, b = v[:, :half], v[:, half:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=1)

    ours = oracle.rope_rows(x, pos, base)
    # the two sides form and reduce the angle (up to pos rad) separately: a few fp64 ulps of it apart
    tol = 1e-12 + 16 * pos * 2.0**-52 * np.abs(x).max()
    np.testing.assert_allclose(half_split(x[:, perm]), ours[:, perm], rtol=0, atol=tol)
    assert np.abs(half_split(x) - ours).max() > 1e-3
