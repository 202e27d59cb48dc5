"""Pure-Python brute force of TPA factor-cache attention, for tiny inputs only.

Written independently of the C oracle to pin it: RoPE is done as complex
multiplication (the RoFormer complex form: pair (x_2j, x_2j+1) is the complex
number x_2j + i x_2j+1 times e^{i p theta_j}, theta_j = base^(-2j/d_h)), the
factor products are scalar loops over the definition K_s[i][c] =
(1/R) sum_r A[s][r][i] B[s][r][c] (TPA notes page, Key design: tensor product
decomposition), and the softmax is computed with ``math.fsum``.
"""
import cmath
import math


def rope_complex(row, pos, base):
    d = len(row)
    out = [0.0] * d
    for j in range(d // 2):
        theta = base ** (-2.0 * j / d)
        z = complex(row[2 * j], row[2 * j + 1]) * cmath.exp(1j * pos * theta)
        out[2 * j], out[2 * j + 1] = z.real, z.imag
    return out


def attention(A_K, B_K, A_V, B_V, kv_pos, q, q_pos, q_nvis, base, scale=None):
    n_kv = len(A_K)
    R_K, h = len(A_K[0]) if n_kv else 0, len(q[0])
    d = len(q[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = []
    for n, qrow in enumerate(q):
        heads = []
        for i in range(h):
            nv = min(q_nvis[n], n_kv)
            if nv <= 0:
                heads.append([0.0] * d)
                continue
            qt = rope_complex(list(qrow[i]), q_pos[n], base)
            z = []
            vals = []
            for s in range(nv):
                R = len(A_K[s])
                k = [math.fsum(A_K[s][r][i] * B_K[s][r][c] for r in range(R)) / R for c in range(d)]
                kt = rope_complex(k, kv_pos[s], base)
                z.append(scale * math.fsum(qt[c] * kt[c] for c in range(d)))
                RV = len(A_V[s])
                vals.append([math.fsum(A_V[s][r][i] * B_V[s][r][c] for r in range(RV)) / RV
                             for c in range(d)])
            M = max(z)
            p = [math.exp(x - M) for x in z]
            L = math.fsum(p)
            heads.append([math.fsum(p[s] * vals[s][c] for s in range(nv)) / L for c in range(d)])
        out.append(heads)
    return out


def query_from_factors(A_Q, B_Q):
    """q[i][c] = (1/R_Q) sum_r A_Q[r][i] B_Q[r][c] for one query token, as fsum loops."""
    RQ, h, d = len(A_Q), len(A_Q[0]), len(B_Q[0])
    return [[math.fsum(A_Q[r][i] * B_Q[r][c] for r in range(RQ)) / RQ for c in range(d)] for i in range(h)]


def scores(A_K, B_K, kv_pos, q_head, q_pos, head, base, scale=None):
    """Scores z_s = scale * rope(q_head, q_pos) . rope(K_s[head], kv_pos[s]) of one query head over every cached
    token, K_s[head][c] = (1/R) sum_r A_K[s][r][head] B_K[s][r][c], as fsum loops."""
    d = len(q_head)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qt = rope_complex(list(q_head), q_pos, base)
    z = []
    for s in range(len(A_K)):
        R = len(A_K[s])
        k = [math.fsum(A_K[s][r][head] * B_K[s][r][c] for r in range(R)) / R for c in range(d)]
        kt = rope_complex(k, kv_pos[s], base)
        z.append(scale * math.fsum(qt[c] * kt[c] for c in range(d)))
    return z
