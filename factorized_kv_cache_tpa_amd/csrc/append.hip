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
// The angle is formed and reduced in fp64; the precision of the rest is
// described at RopeMath.  The result is rounded once to the storage type.
// This is an HBM copy of one token per sequence per decode step; its cost is
// latency (a position load, the angle table, the stores), so every input
// load is issued first and query rows are spread over several work-groups.
#include "common.h"

namespace tpa {
namespace {

// cos and sin of pos * theta_j for the d_h/2 pairs of one position, shared by the work-group.
// theta is this thread's theta_j (j = threadIdx.x < d_h/2; d_h/2 <= kAppendThreads), loaded up front.
template <typename T>
__device__ inline void rope_table(typename RopeMath<T>::F *cs, int d_h, double pos, double theta) {
    const int j = threadIdx.x;
    if (j < d_h / 2) rope_cos_sin<T>(cs + 2 * j, pos, theta);
    __syncthreads();
}

// Two adjacent elements (a rotary pair) moved as one load or store.
template <typename T>
struct Pair;
template <>
struct Pair<uint16_t> {
    using V = uint32_t;
    __device__ static V zero() { return 0u; }
    __device__ static float lo(V v) { return bf16_to_f32(uint16_t(v & 0xffffu)); }
    __device__ static float hi(V v) { return bf16_to_f32(uint16_t(v >> 16)); }
    __device__ static V make(float a, float b) { return pack_bf16x2(a, b); }
    __device__ static uint16_t first(V v) { return uint16_t(v & 0xffffu); }
    __device__ static uint16_t second(V v) { return uint16_t(v >> 16); }
};
template <>
struct Pair<float> {
    using V = float2;
    __device__ static V zero() { return make_float2(0.f, 0.f); }
    __device__ static double lo(V v) { return double(v.x); }
    __device__ static double hi(V v) { return double(v.y); }
    __device__ static V make(double a, double b) { return make_float2(float(a), float(b)); }
    __device__ static float first(V v) { return v.x; }
    __device__ static float second(V v) { return v.y; }
};

// (x0, x1) rotated by the angle whose cos, sin sit at cs[2j], cs[2j+1]; one rounding to T at the end.
template <typename T>
__device__ inline typename Pair<T>::V rope_pair(typename Pair<T>::V x, const typename RopeMath<T>::F *cs, int j) {
    using P = Pair<T>;
    typename RopeMath<T>::F y0, y1;
    rope_rotate(P::lo(x), P::hi(x), cs[2 * j], cs[2 * j + 1], y0, y1);
    return P::make(y0, y1);
}

template <typename T>
__device__ inline T zero_of() { return T(0); }

// Per-thread register budget of one work-group.  A token's factors span at most RH * DP / 2 <= 512
// rotary pairs and RH * HP <= 256 head-factor values.  Query rows are split over work-groups of
// kQPairs pairs per thread.  Every load is issued before the angle table is built, so the memory
// latency of the inputs overlaps the table instead of following it.
constexpr int kKvPairs = 4;
constexpr int kKvGates = 2;
constexpr int kQPairs = 4;

}  // namespace

int64_t append_q_groups(int q_rows, int d_h) {
    const int64_t per_group = int64_t(kAppendThreads) * kQPairs;
    return (int64_t(q_rows) * (d_h / 2) + per_group - 1) / per_group;
}

namespace {

// Inverse scales of A_K, B_K, A_V, B_V for an E4M3 cache (code = E4M3(value * inv)).
struct InvScale {
    float v[4];
};

// Grid: one work-group per cache token (n < n_kv), then append_q_groups(q_rows, d_h) work-groups per
// query token, each rotating kAppendThreads * kQPairs consecutive pairs of that token's rows.
// kF8: bf16 inputs, E4M3 cache (cache_raw holds bytes); otherwise the cache holds T.
template <typename T, bool kF8>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    Layout L, int h, int d_h, int RK, int RV, RopeTable rt, void *__restrict__ cache_raw, int64_t capacity,
    int64_t n_kv, const int64_t *__restrict__ slot, const int32_t *__restrict__ kv_pos, const T *__restrict__ A_K,
    const T *__restrict__ B_K, const T *__restrict__ A_V, const T *__restrict__ B_V, int64_t n_q, int q_rows,
    int q_groups, const int32_t *__restrict__ q_pos, const T *q_in, T *q_out, InvScale inv) {
    using P = Pair<T>;
    using V = typename P::V;
    using F = typename RopeMath<T>::F;
    __shared__ F cs[256];  // cos, sin per rotary pair (d_h <= 256)
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const double theta = tid < d_h / 2 ? rt.theta[tid] : 0.0;
    if (n < n_kv) {
        const int64_t s = slot[n];
        const double pos = double(kv_pos[n]);
        const int HD = L.DP / 2;  // pairs per padded feature row
        V kx[kKvPairs], vx[kKvPairs];
        T ga[kKvGates], gv[kKvGates];
#pragma unroll
        for (int k = 0; k < kKvPairs; ++k) {
            const int idx = tid + k * kAppendThreads, r = idx / HD, d = 2 * (idx % HD);
            const bool in = idx < L.RH * HD && d < d_h;
            kx[k] = in && r < RK ? *reinterpret_cast<const V *>(B_K + (n * RK + r) * d_h + d) : P::zero();
            vx[k] = in && r < RV ? *reinterpret_cast<const V *>(B_V + (n * RV + r) * d_h + d) : P::zero();
        }
#pragma unroll
        for (int k = 0; k < kKvGates; ++k) {
            const int idx = tid + k * kAppendThreads, r = idx / L.HP, i = idx % L.HP;
            const bool in = idx < L.RH * L.HP && i < h;
            ga[k] = in && r < RK ? A_K[(n * RK + r) * h + i] : zero_of<T>();
            gv[k] = in && r < RV ? A_V[(n * RV + r) * h + i] : zero_of<T>();
        }
        rope_table<T>(cs, d_h, pos, theta);
        if (s < 0 || s >= capacity) return;  // uniform over the work-group, after the barrier
        const int TOK = L.tok_per_block();
        const int row0 = int(s % TOK) * L.RH;
        if constexpr (kF8) {
            // E4M3 record: every element is the code of its fp32 value times the inverse scale; B_K's pair
            // is rotated in fp32 first (one rounding, straight to the code).  Padded rows and heads: code 0.
            uint8_t *blk = reinterpret_cast<uint8_t *>(cache_raw) + (s / TOK) * L.block_elems();
#pragma unroll
            for (int k = 0; k < kKvGates; ++k) {
                const int idx = tid + k * kAppendThreads, r = idx / L.HP, i = idx % L.HP;
                if (idx < L.RH * L.HP) {
                    const int off = L.gate(row0 + r, i);
                    blk[L.off_ak() + off] = e4m3_one(Elem<T>::to_f32(ga[k]) * inv.v[0]);
                    blk[L.off_av() + off] = e4m3_one(Elem<T>::to_f32(gv[k]) * inv.v[2]);
                }
            }
#pragma unroll
            for (int k = 0; k < kKvPairs; ++k) {
                const int idx = tid + k * kAppendThreads, r = idx / HD, j = idx % HD, d = 2 * j;
                if (idx < L.RH * HD) {
                    float y0 = 0.f, y1 = 0.f;
                    if (r < RK && d < d_h) rope_rotate(P::lo(kx[k]), P::hi(kx[k]), cs[2 * j], cs[2 * j + 1], y0, y1);
                    // d even: d and d + 1 are adjacent bytes of one lane's 8-code run
                    *reinterpret_cast<uint16_t *>(blk + L.off_bk() + L.bk(row0 + r, d)) =
                        uint16_t(e4m3_pair(y0 * inv.v[1], y1 * inv.v[1]));
                    const uint32_t vc = e4m3_pair(P::lo(vx[k]) * inv.v[3], P::hi(vx[k]) * inv.v[3]);
                    blk[L.off_bv() + L.bv(row0 + r, d)] = uint8_t(vc & 0xffu);
                    blk[L.off_bv() + L.bv(row0 + r, d + 1)] = uint8_t(vc >> 8);
                }
            }
            return;
        }
        T *blk = reinterpret_cast<T *>(cache_raw) + (s / TOK) * L.block_elems();
#pragma unroll
        for (int k = 0; k < kKvGates; ++k) {
            const int idx = tid + k * kAppendThreads, r = idx / L.HP, i = idx % L.HP;
            if (idx < L.RH * L.HP) {
                const int off = L.gate(row0 + r, i);
                blk[L.off_ak() + off] = ga[k];
                blk[L.off_av() + off] = gv[k];
            }
        }
#pragma unroll
        for (int k = 0; k < kKvPairs; ++k) {
            const int idx = tid + k * kAppendThreads, r = idx / HD, j = idx % HD, d = 2 * j;
            if (idx < L.RH * HD) {
                const V y = r < RK && d < d_h ? rope_pair<T>(kx[k], cs, j) : P::zero();
                T *pk = blk + L.off_bk() + L.bk(row0 + r, d);
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<V *>(pk) = y;  // bf16: d even, so d, d+1 share one lane's 8-value k-run
                } else {
                    pk[0] = P::first(y);
                    blk[L.off_bk() + L.bk(row0 + r, d + 1)] = P::second(y);
                }
                blk[L.off_bv() + L.bv(row0 + r, d)] = P::first(vx[k]);
                blk[L.off_bv() + L.bv(row0 + r, d + 1)] = P::second(vx[k]);
            }
        }
    } else {
        const int64_t g = n - n_kv;
        const int64_t nq = g / q_groups;
        if (nq >= n_q) return;  // uniform over the work-group
        const double pos = double(q_pos[nq]);
        const int HD = d_h / 2;
        const int items = q_rows * HD;  // pair idx = row * HD + j sits at element 2 * idx of the token
        const int first = int(g % q_groups) * (kAppendThreads * kQPairs);
        const V *src = reinterpret_cast<const V *>(q_in + nq * q_rows * d_h);
        V *dst = reinterpret_cast<V *>(q_out + nq * q_rows * d_h);
        V x[kQPairs];
#pragma unroll
        for (int k = 0; k < kQPairs; ++k) {
            const int idx = first + k * kAppendThreads + tid;
            x[k] = idx < items ? src[idx] : P::zero();
        }
        rope_table<T>(cs, d_h, pos, theta);
#pragma unroll
        for (int k = 0; k < kQPairs; ++k) {
            const int idx = first + k * kAppendThreads + tid;
            if (idx < items) dst[idx] = rope_pair<T>(x[k], cs, idx % HD);
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

RopeTable make_rope_table(int d_h, double base) {
    RopeTable rt;
    for (int j = 0; j < 128; ++j) rt.theta[j] = j < d_h / 2 ? pow(base, -2.0 * double(j) / double(d_h)) : 0.0;
    return rt;
}

hipError_t launch_append(const Layout &L, int h, int d_h, int RK, int RV, double base, void *cache,
                         int64_t capacity, int64_t n_kv, const int64_t *slot, const int32_t *kv_pos,
                         const void *A_K, const void *B_K, const void *A_V, const void *B_V, int64_t n_q,
                         int q_rows, const int32_t *q_pos, const void *q_in, void *q_out, const float *inv_scale,
                         hipStream_t s) {
    if (L.RH * L.DP / 2 > kKvPairs * kAppendThreads || L.RH * L.HP > kKvGates * kAppendThreads ||
        d_h / 2 > kAppendThreads)
        return hipErrorInvalidValue;  // outside the validated dimension range
    const int64_t q_groups = n_q > 0 ? append_q_groups(q_rows, d_h) : 1;
    const int64_t grid = n_kv + n_q * q_groups;
    if (grid == 0) return hipSuccess;
    if (grid > int64_t(0x7fffffff)) return hipErrorInvalidConfiguration;
    const RopeTable rt = make_rope_table(d_h, base);
    InvScale inv;
    for (int k = 0; k < 4; ++k) inv.v[k] = inv_scale ? inv_scale[k] : 1.f;
    if (L.f8) {
        using T = uint16_t;
        hipLaunchKernelGGL((append_kernel<T, true>), dim3(unsigned(grid)), dim3(kAppendThreads), 0, s, L, h, d_h, RK,
                           RV, rt, cache, capacity, n_kv, slot, kv_pos, (const T *)A_K, (const T *)B_K,
                           (const T *)A_V, (const T *)B_V, n_q, q_rows, int(q_groups), q_pos, (const T *)q_in,
                           (T *)q_out, inv);
    } else if (L.es == 2) {
        using T = uint16_t;
        hipLaunchKernelGGL((append_kernel<T, false>), dim3(unsigned(grid)), dim3(kAppendThreads), 0, s, L, h, d_h,
                           RK, RV, rt, cache, capacity, n_kv, slot, kv_pos, (const T *)A_K, (const T *)B_K,
                           (const T *)A_V, (const T *)B_V, n_q, q_rows, int(q_groups), q_pos, (const T *)q_in,
                           (T *)q_out, inv);
    } else {
        using T = float;
        hipLaunchKernelGGL((append_kernel<T, false>), dim3(unsigned(grid)), dim3(kAppendThreads), 0, s, L, h, d_h,
                           RK, RV, rt, cache, capacity, n_kv, slot, kv_pos, (const T *)A_K, (const T *)B_K,
                           (const T *)A_V, (const T *)B_V, n_q, q_rows, int(q_groups), q_pos, (const T *)q_in,
                           (T *)q_out, inv);
    }
    return hipGetLastError();
}

hipError_t launch_read(const Layout &L, int h, int d_h, int RK, int RV, const void *cache, int64_t capacity,
                       int64_t n, const int64_t *slot, void *A_K, void *B_K, void *A_V, void *B_V,
                       hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (L.f8) {
        using T = uint8_t;
        hipLaunchKernelGGL(read_kernel<T>, dim3(unsigned(n)), dim3(kAppendThreads), 0, s, L, h, d_h, RK, RV,
                           (const T *)cache, capacity, slot, (T *)A_K, (T *)B_K, (T *)A_V, (T *)B_V);
    } else if (L.es == 2) {
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
