// Cache append with RoPE on the key feature factor, query rotation, and cache read-back.
//
// TPA notes page, Key design, RoPE compatibility (Theorem 3.1): the rotary
// operator acts on the feature factor B only, so rotating B_K once when a
// token enters the cache keeps the relative-position property of the scores;
// A_K, A_V and B_V are stored unchanged.  Query rows (a full query, or a B_Q
// factor) are rotated by the same operator at their own positions.
//
// Rotation: RoFormer pairs (2j, 2j+1), theta_j = base^(-2j/d_h),
// (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a), a = pos * theta_j.
// The angle and the rotation are computed in fp64 (positions reach 131072
// and beyond, where an fp32 angle is off by milliradians) and the result is
// rounded once to the storage type.  This is an HBM copy, not on the
// per-token hot loop.
#include "common.h"

namespace tpa {
namespace {

constexpr int kAppendThreads = 128;

// cos and sin of pos * theta_j for the d_h/2 pairs of one position, fp64, shared by the work-group.
// The angle is reduced modulo 2 pi first (Cody-Waite with 2 pi split in two doubles; positions are
// int32, so |angle| < 2^31 and the two-part split keeps r exact to ~1e-15), so sincos sees |r| <= pi.
__device__ inline void rope_table(double *cs, int d_h, double pos, const RopeTable &rt) {
    constexpr double kTwoPiHi = 6.283185307179586232;    // nearest double to 2 pi
    constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2 pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    for (int j = threadIdx.x; j < d_h / 2; j += blockDim.x) {
        const double phi = pos * rt.theta[j];
        const double k = rint(phi * kInvTwoPi);
        const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, phi));
        double sn, cn;
        sincos(r, &sn, &cn);
        cs[2 * j] = cn;
        cs[2 * j + 1] = sn;
    }
    __syncthreads();
}

template <typename T>
__device__ inline void rope_pair(T x0, T x1, const double *cs, int j, T &y0, T &y1) {
    const double c = cs[2 * j], s = cs[2 * j + 1];
    const double a = double(Elem<T>::to_f32(x0)), b = double(Elem<T>::to_f32(x1));
    y0 = Elem<T>::from_f64(a * c - b * s);
    y1 = Elem<T>::from_f64(a * s + b * c);
}

template <typename T>
__device__ inline T zero_of() { return T(0); }

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    Layout L, int h, int d_h, int RK, int RV, RopeTable rt, T *__restrict__ cache, int64_t capacity, int64_t n_kv,
    const int64_t *__restrict__ slot, const int32_t *__restrict__ kv_pos, const T *__restrict__ A_K,
    const T *__restrict__ B_K, const T *__restrict__ A_V, const T *__restrict__ B_V, int64_t n_q, int q_rows,
    const int32_t *__restrict__ q_pos, const T *q_in, T *q_out) {
    __shared__ double cs[256];  // cos, sin per rotary pair (d_h <= 256)
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    if (n < n_kv) {
        const int64_t s = slot[n];
        if (s < 0 || s >= capacity) return;
        const int TOK = L.tok_per_block();
        T *blk = cache + (s / TOK) * L.block_elems();
        const int row0 = int(s % TOK) * L.RH;
        rope_table(cs, d_h, double(kv_pos[n]), rt);
        // head factors: gates stored per (row, head)
        for (int idx = tid; idx < L.RH * L.HP; idx += kAppendThreads) {
            const int r = idx / L.HP, i = idx % L.HP;
            const int off = L.gate(row0 + r, i);
            blk[L.off_ak() + off] = (r < RK && i < h) ? A_K[(n * RK + r) * h + i] : zero_of<T>();
            blk[L.off_av() + off] = (r < RV && i < h) ? A_V[(n * RV + r) * h + i] : zero_of<T>();
        }
        // feature factors: B_K rotated pairwise, B_V copied
        const int HD = L.DP / 2;
        for (int idx = tid; idx < L.RH * HD; idx += kAppendThreads) {
            const int r = idx / HD, j = idx % HD, d = 2 * j;
            T k0 = zero_of<T>(), k1 = zero_of<T>(), v0 = zero_of<T>(), v1 = zero_of<T>();
            if (r < RK && d < d_h) {
                const T *src = B_K + (n * RK + r) * d_h + d;
                rope_pair<T>(src[0], src[1], cs, j, k0, k1);
            }
            if (r < RV && d < d_h) {
                const T *src = B_V + (n * RV + r) * d_h + d;
                v0 = src[0];
                v1 = src[1];
            }
            blk[L.off_bk() + L.bk(row0 + r, d)] = k0;
            blk[L.off_bk() + L.bk(row0 + r, d + 1)] = k1;
            blk[L.off_bv() + L.bv(row0 + r, d)] = v0;
            blk[L.off_bv() + L.bv(row0 + r, d + 1)] = v1;
        }
    } else {
        const int64_t nq = n - n_kv;
        if (nq >= n_q) return;
        rope_table(cs, d_h, double(q_pos[nq]), rt);
        const int HD = d_h / 2;
        for (int idx = tid; idx < q_rows * HD; idx += kAppendThreads) {
            const int row = idx / HD, j = idx % HD;
            const int64_t o = (nq * q_rows + row) * d_h + 2 * j;
            const T x0 = q_in[o], x1 = q_in[o + 1];
            T y0, y1;
            rope_pair<T>(x0, x1, cs, j, y0, y1);
            q_out[o] = y0;
            q_out[o + 1] = y1;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void read_kernel(Layout L, int h, int d_h, int RK, int RV,
                                                             const T *__restrict__ cache, int64_t capacity,
                                                             const int64_t *__restrict__ slot, T *A_K, T *B_K,
                                                             T *A_V, T *B_V) {
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t s = slot[n];
    const bool ok = s >= 0 && s < capacity;
    const int TOK = L.tok_per_block();
    const T *blk = cache + (ok ? (s / TOK) * L.block_elems() : 0);
    const int row0 = ok ? int(s % TOK) * L.RH : 0;
    for (int idx = tid; idx < RK * h; idx += kAppendThreads) {
        const int r = idx / h, i = idx % h;
        A_K[(n * RK + r) * h + i] = ok ? blk[L.off_ak() + L.gate(row0 + r, i)] : zero_of<T>();
    }
    for (int idx = tid; idx < RV * h; idx += kAppendThreads) {
        const int r = idx / h, i = idx % h;
        A_V[(n * RV + r) * h + i] = ok ? blk[L.off_av() + L.gate(row0 + r, i)] : zero_of<T>();
    }
    for (int idx = tid; idx < RK * d_h; idx += kAppendThreads) {
        const int r = idx / d_h, d = idx % d_h;
        B_K[(n * RK + r) * d_h + d] = ok ? blk[L.off_bk() + L.bk(row0 + r, d)] : zero_of<T>();
    }
    for (int idx = tid; idx < RV * d_h; idx += kAppendThreads) {
        const int r = idx / d_h, d = idx % d_h;
        B_V[(n * RV + r) * d_h + d] = ok ? blk[L.off_bv() + L.bv(row0 + r, d)] : zero_of<T>();
    }
}

}  // namespace

hipError_t launch_append(const Layout &L, int h, int d_h, int RK, int RV, double base, void *cache,
                         int64_t capacity, int64_t n_kv, const int64_t *slot, const int32_t *kv_pos,
                         const void *A_K, const void *B_K, const void *A_V, const void *B_V, int64_t n_q,
                         int q_rows, const int32_t *q_pos, const void *q_in, void *q_out, hipStream_t s) {
    const int64_t grid = n_kv + n_q;
    if (grid == 0) return hipSuccess;
    RopeTable rt;
    for (int j = 0; j < 128; ++j) rt.theta[j] = j < d_h / 2 ? pow(base, -2.0 * double(j) / double(d_h)) : 0.0;
    if (L.es == 2) {
        using T = uint16_t;
        hipLaunchKernelGGL(append_kernel<T>, dim3(unsigned(grid)), dim3(kAppendThreads), 0, s, L, h, d_h, RK, RV,
                           rt, (T *)cache, capacity, n_kv, slot, kv_pos, (const T *)A_K, (const T *)B_K,
                           (const T *)A_V, (const T *)B_V, n_q, q_rows, q_pos, (const T *)q_in, (T *)q_out);
    } else {
        using T = float;
        hipLaunchKernelGGL(append_kernel<T>, dim3(unsigned(grid)), dim3(kAppendThreads), 0, s, L, h, d_h, RK, RV,
                           rt, (T *)cache, capacity, n_kv, slot, kv_pos, (const T *)A_K, (const T *)B_K,
                           (const T *)A_V, (const T *)B_V, n_q, q_rows, q_pos, (const T *)q_in, (T *)q_out);
    }
    return hipGetLastError();
}

hipError_t launch_read(const Layout &L, int h, int d_h, int RK, int RV, const void *cache, int64_t capacity,
                       int64_t n, const int64_t *slot, void *A_K, void *B_K, void *A_V, void *B_V,
                       hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (L.es == 2) {
        using T = uint16_t;
        hipLaunchKernelGGL(read_kernel<T>, dim3(unsigned(n)), dim3(kAppendThreads), 0, s, L, h, d_h, RK, RV,
                           (const T *)cache, capacity, slot, (T *)A_K, (T *)B_K, (T *)A_V, (T *)B_V);
    } else {
        using T = float;
        hipLaunchKernelGGL(read_kernel<T>, dim3(unsigned(n)), dim3(kAppendThreads), 0, s, L, h, d_h, RK, RV,
                           (const T *)cache, capacity, slot, (T *)A_K, (T *)B_K, (T *)A_V, (T *)B_V);
    }
    return hipGetLastError();
}

}  // namespace tpa
