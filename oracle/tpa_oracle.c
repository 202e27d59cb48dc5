/*
 * tpa_oracle.c -- fp64 CPU oracle for attention over a Tensor Product Attention
 * (TPA) factor cache.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark call it; the library never does, and it shares
 * no code, header, table or helper with the HIP path.
 *
 * It computes the plain definition of the result, step by step, with nothing
 * blocked, fused or reordered beyond what the definition states:
 *
 *   1. Factor materialization ("Tensor Product Attention Is All You Need",
 *      notes page, Key design: tensor product decomposition):
 *          K_s = (1/R_K) * A_K[s]^T * B_K[s]      (h x d_h)
 *          V_s = (1/R_V) * A_V[s]^T * B_V[s]      (h x d_h)
 *      with A in R^{R x h} (head factor) and B in R^{R x d_h} (feature
 *      factor).  Done one head row at a time, in fp64, from the unrotated
 *      factors.
 *   2. Standard rotary position embedding applied to the *full* key rows and
 *      to the query rows (same page, Key design: RoPE compatibility,
 *      Theorem 3.1, which states the rotation is a relative-position operator
 *      T_{t-s}).  Convention (the pages print only T_{t-s}): RoFormer pairs
 *      (2j, 2j+1), theta_j = base^(-2j/d_h), a pair (x0, x1) at position p
 *      maps to (x0 cos(p theta_j) - x1 sin(p theta_j),
 *               x0 sin(p theta_j) + x1 cos(p theta_j)).
 *   3. Textbook scaled dot-product softmax attention, per query row and head:
 *          z_s = scale * <q~_i, K~_s[i,:]>,  M = max_s z_s,
 *          p_s = exp(z_s - M), out_i = sum_s p_s V_s[i,:] / sum_s p_s
 *      over the cached tokens the query sees (the first q_nvis[n] tokens;
 *      a query that sees none returns zeros).  The pages print no softmax
 *      scale; the caller passes it (1/sqrt(d_h) is the textbook choice).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Step 2: rotate one row of d values (d even) to position pos in place. */
void tpa_oracle_rope_row(double *x, int d, double pos, double base) {
    for (int j = 0; j < d / 2; ++j) {
        double theta = pow(base, -2.0 * (double)j / (double)d);
        double phi = pos * theta;
        double c = cos(phi), s = sin(phi);
        double x0 = x[2 * j], x1 = x[2 * j + 1];
        x[2 * j] = x0 * c - x1 * s;
        x[2 * j + 1] = x0 * s + x1 * c;
    }
}

/* Step 2 for many rows at once: row k of x (d values) rotated to position pos[k] in place, each row exactly as
 * tpa_oracle_rope_row rotates it (a loop over rows, nothing shared between them). */
void tpa_oracle_rope_rows(double *x, int64_t n_rows, int d, const double *pos, double base, int n_threads) {
    if (n_threads < 1) n_threads = 1;
#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t k = 0; k < n_rows; ++k) tpa_oracle_rope_row(x + k * d, d, pos[k], base);
}

/* Step 1 for one head row i of one token: row = (1/R) sum_r A[r][i] * B[r][:]. */
static void materialize_row(double *row, int h, int d, int R, const double *A /* [R][h] */,
                            const double *B /* [R][d] */, int i) {
    for (int c = 0; c < d; ++c) row[c] = 0.0;
    for (int r = 0; r < R; ++r) {
        double a = A[(int64_t)r * h + i];
        for (int c = 0; c < d; ++c) row[c] += a * B[(int64_t)r * d + c];
    }
    for (int c = 0; c < d; ++c) row[c] /= (double)R;
}

/*
 * Attention of n_q query rows over n_kv cached tokens.
 *   AK [n_kv][RK][h], BK [n_kv][RK][d], AV [n_kv][RV][h], BV [n_kv][RV][d]  unrotated factors
 *   kv_pos [n_kv]                       position of each cached token
 *   q [n_q][h][d], q_pos [n_q]           unrotated query rows and their positions
 *   q_nvis [n_q]                        query n sees cached tokens 0 .. q_nvis[n]-1
 *   out [n_q][h][d]
 * Returns 0, or -1 on a bad argument.
 */
int tpa_oracle_attention(int h, int d, int RK, int RV, int64_t n_kv, const double *AK,
                         const double *BK, const double *AV, const double *BV,
                         const double *kv_pos, int64_t n_q, const double *q,
                         const double *q_pos, const int64_t *q_nvis, double base, double scale,
                         double *out, int n_threads) {
    if (h < 1 || d < 2 || (d & 1) || RK < 1 || RV < 1 || n_kv < 0 || n_q < 0) return -1;
    if (n_threads < 1) n_threads = 1;
    int bad = 0;

#pragma omp parallel for schedule(dynamic) num_threads(n_threads) reduction(| : bad)
    for (int i = 0; i < h; ++i) {
        /* materialized, rotated key rows and value rows of head i for every cached token */
        double *Kt = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1) * d);
        double *Vt = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1) * d);
        double *z = (double *)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
        double *qt = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!Kt || !Vt || !z || !qt || !acc) {
            bad = 1;
        } else {
            for (int64_t s = 0; s < n_kv; ++s) {
                materialize_row(Kt + s * d, h, d, RK, AK + s * RK * h, BK + s * RK * d, i);
                tpa_oracle_rope_row(Kt + s * d, d, kv_pos[s], base);
                materialize_row(Vt + s * d, h, d, RV, AV + s * RV * h, BV + s * RV * d, i);
            }
            for (int64_t n = 0; n < n_q; ++n) {
                double *o = out + (n * h + i) * d;
                int64_t nv = q_nvis[n] < n_kv ? q_nvis[n] : n_kv;
                if (nv <= 0) {
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    continue;
                }
                memcpy(qt, q + (n * h + i) * d, sizeof(double) * (size_t)d);
                tpa_oracle_rope_row(qt, d, q_pos[n], base);
                /* pass 1: scores and their maximum */
                double M = -INFINITY;
                for (int64_t s = 0; s < nv; ++s) {
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c) dot += qt[c] * Kt[s * d + c];
                    z[s] = scale * dot;
                    if (z[s] > M) M = z[s];
                }
                /* pass 2: normalized weights applied to the value rows */
                double L = 0.0;
                for (int c = 0; c < d; ++c) acc[c] = 0.0;
                for (int64_t s = 0; s < nv; ++s) {
                    double p = exp(z[s] - M);
                    L += p;
                    for (int c = 0; c < d; ++c) acc[c] += p * Vt[s * d + c];
                }
                for (int c = 0; c < d; ++c) o[c] = acc[c] / L;
            }
        }
        free(Kt);
        free(Vt);
        free(z);
        free(qt);
        free(acc);
    }
    return bad ? -1 : 0;
}

/* Query rows from query factors (full TPA: the tensor product decomposition applied to Q, same page,
 * Key design: tensor product decomposition):  q[n][i][c] = (1/R_Q) sum_r A_Q[n][r][i] B_Q[n][r][c],
 * A_Q [n][R_Q][h], B_Q [n][R_Q][d] (unrotated), out [n][h][d].  The result is the query of step 3 above,
 * rotated there at its position like any other query row. */
void tpa_oracle_query_from_factors(int h, int d, int RQ, int64_t n, const double *AQ, const double *BQ,
                                   double *out) {
    for (int64_t t = 0; t < n; ++t)
        for (int i = 0; i < h; ++i)
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int r = 0; r < RQ; ++r) acc += AQ[(t * RQ + r) * h + i] * BQ[(t * RQ + r) * d + c];
                out[(t * h + i) * d + c] = acc / RQ;
            }
}

/* ---- 8-bit factor storage (the pages' next step: TPA combined with low-bit storage, which they call
 * unexplored; parity unpinned as a method, the codec itself is pinned).  Reading: every factor element is
 * stored as an OCP 8-bit floating-point E4M3 code of (value / scale), one fixed scale per factor tensor;
 * the stored value is code * scale.  E4M3 per the OCP 8-bit floating point specification: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal, m * 2^-9; exponent field
 * e > 0 is 2^(e-7) * (1 + m/8); there are no infinities and only S.1111.111 is NaN, so the largest finite
 * magnitude is 448 (S.1111.110).  The oracle's steps then run on the decoded values exactly as on any
 * other factors. */
double tpa_oracle_e4m3_decode(uint8_t code) {
    const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest code by brute force over the 127 non-negative finite codes, ties to the code with the even
 * mantissa (round to nearest even); magnitudes above 448 saturate to 448; the sign is kept (so -0.0 and
 * negative values below half the smallest subnormal give 0x80); NaN gives 0x7F. */
uint8_t tpa_oracle_e4m3_encode(double x) {
    if (isnan(x)) return 0x7F;
    const int neg = signbit(x) != 0;
    const double a = fabs(x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 126; ++c) {
        const double err = fabs(a - tpa_oracle_e4m3_decode((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (neg ? 0x80 : 0));
}

void tpa_oracle_e4m3_decode_n(int64_t n, const uint8_t *codes, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = tpa_oracle_e4m3_decode(codes[i]);
}

void tpa_oracle_e4m3_encode_n(int64_t n, const double *x, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = tpa_oracle_e4m3_encode(x[i]);
}

/* Per-token element counts the pages compare (tensor product decomposition paragraph):
 * a TPA cache holds (R_K + R_V)(h + d_h) elements per token, a dense MHA cache 2 h d_h. */
int64_t tpa_oracle_factor_elems_per_token(int h, int d, int RK, int RV) {
    return (int64_t)(RK + RV) * (int64_t)(h + d);
}

int64_t tpa_oracle_dense_elems_per_token(int h, int d) { return 2 * (int64_t)h * (int64_t)d; }

int tpa_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
