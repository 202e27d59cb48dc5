// Causal chunked prefill over a TPA factor cache.
//
// TPA notes page, Key design: K_s = (1/R_K) A_K[s]^T B_K[s] and V_s likewise;
// FlashTPA: no full K/V in device memory.  A prefill chunk has many query
// rows per head, so each work-group rebuilds one head's key and value rows of
// a 32-token tile on chip,
//     K~_i[s,:] = sum_r A_K[s,r,i] B~_K[s,r,:]      (1/R_K folded into the scale)
//     V_i[s,:]  = sum_r A_V[s,r,i] B_V[s,r,:]       (1/R_V applied at the end)
// in fp32 from the cached factors, rounds them once to bf16 into LDS, and
// runs a flash-attention loop on the bf16 matrix cores (32x32x16):
//     S^T = K~_i Q~^T   (M = keys, N = queries, K = d_h)
//     causal mask: chunk row j (position ctx + j) sees keys 0 .. ctx + j
//     online softmax per query (a lane owns one query column)
//     O^T += V_i^T P^T  (M = d_h, N = queries, K = keys)
// The key order inside the value contraction is permuted to match the score
// accumulator layout, so P never leaves the lane that computed it.
#include "common.h"

namespace tpa {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kQT = 32 * kPrefillWaves;  // query rows per work-group
constexpr int kKT = 32;                  // keys per tile

__device__ __forceinline__ floatx16 mma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    uint4 v;
    v.x = uint32_t(f32_to_bf16_rne(x[0])) | (uint32_t(f32_to_bf16_rne(x[1])) << 16);
    v.y = uint32_t(f32_to_bf16_rne(x[2])) | (uint32_t(f32_to_bf16_rne(x[3])) << 16);
    v.z = uint32_t(f32_to_bf16_rne(x[4])) | (uint32_t(f32_to_bf16_rne(x[5])) << 16);
    v.w = uint32_t(f32_to_bf16_rne(x[6])) | (uint32_t(f32_to_bf16_rne(x[7])) << 16);
    return __builtin_bit_cast(bf16x8, v);
}

template <int HP, int DP, int RH>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
    constexpr int KS = DP / 16;  // score K steps
    constexpr int MB = DP / 32;  // value M blocks
    constexpr int TOK = kRows / RH;
    constexpr int SKS = DP + 8;   // LDS row stride of K~ (bf16 elements)
    constexpr int SVS = kKT + 8;  // LDS row stride of V^T
    __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * SKS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[DP * SVS];
    const Layout L = {HP, DP, RH, 8, 2};
    const int64_t BLK = L.block_elems();

    const int head = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 31, hi = lane >> 5;
    const int j0 = blockIdx.x * kQT;
    const int jw = j0 + 32 * w;  // first query row of this wave
    const int jq = jw + col;     // query row of this lane's accumulator column
    int ctx = p.ctx_len[b];
    ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
    const int64_t start = p.seq_start[b];
    float *out = p.out + int64_t(b) * p.chunk * p.h * p.d_h;

    if (start < 0 || start % TOK != 0) {  // misaligned sequence: report NaN
        for (int idx = tid; idx < kQT * p.d_h; idx += kPrefillThreads) {
            const int j = j0 + idx / p.d_h, d = idx % p.d_h;
            if (j < p.chunk) out[(int64_t(j) * p.h + head) * p.d_h + d] = __builtin_nanf("");
        }
        return;
    }
    const uint16_t *seq = reinterpret_cast<const uint16_t *>(p.cache) + (start / TOK) * BLK;

    // Q operand (B of S^T): lane supplies Q~[jq][16 ks + 8 hi + e]
    bf16x8 qf[KS];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) + (int64_t(b) * p.chunk + jq) * p.h * p.d_h +
                               int64_t(head) * p.d_h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 16 * ks + 8 * hi + e;
                x[e] = (jq < p.chunk && d < p.d_h) ? bf16_to_f32(qrow[d]) : 0.f;
            }
            qf[ks] = pack8(x);
        }
    }

    floatx16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][v] = 0.f;
    float run_m = -INFINITY, run_l = 0.f;

    const int j_last = min(p.chunk, j0 + kQT) - 1;
    const int n_keys = ctx + j_last + 1;  // keys any row of this work-group sees
    const int wave_last = min(p.chunk - 1, jw + 31);
    const int n_kt = (n_keys + kKT - 1) / kKT;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int key0 = kt * kKT;
        // ---- rebuild K~_i and V_i of this tile (fp32 math, one bf16 rounding)
        for (int idx = tid; idx < kKT * (DP / 8); idx += kPrefillThreads) {
            const int k = idx / (DP / 8), d0 = 8 * (idx % (DP / 8));
            const int key = key0 + k;
            float kv[8], vv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[e] = vv[e] = 0.f;
            if (key < n_keys) {
                const uint16_t *blk = seq + int64_t(key / TOK) * BLK;
                const int row0 = (key % TOK) * RH;
                for (int r = 0; r < p.RK; ++r) {
                    const float a = bf16_to_f32(blk[L.off_ak() + L.gate(row0 + r, head)]);
                    const uint4 raw = *reinterpret_cast<const uint4 *>(blk + L.off_bk() + L.bk(row0 + r, d0));
                    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t h16 = (e & 1) ? (wds[e >> 1] & 0xffff0000u) : (wds[e >> 1] << 16);
                        kv[e] += a * __uint_as_float(h16);
                    }
                }
                for (int r = 0; r < p.RV; ++r) {
                    const float a = bf16_to_f32(blk[L.off_av() + L.gate(row0 + r, head)]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) vv[e] += a * bf16_to_f32(blk[L.off_bv() + L.bv(row0 + r, d0 + e)]);
                }
            }
            const bf16x8 kp = pack8(kv);
            *reinterpret_cast<bf16x8 *>(&sK[k * SKS + d0]) = kp;
#pragma unroll
            for (int e = 0; e < 8; ++e) sV[(d0 + e) * SVS + k] = f32_to_bf16_rne(vv[e]);
        }
        __syncthreads();

        if (jw < p.chunk && key0 <= ctx + wave_last) {
            // ---- S^T = K~ Q~^T
            floatx16 s;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sK[col * SKS + 16 * ks + 8 * hi]);
                s = mma32(a, qf[ks], s);
            }
            // ---- causal mask, online softmax (log2 units)
            float z[16];
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = key0 + 8 * (v >> 2) + 4 * hi + (v & 3);
                const bool vis = jq < p.chunk && key <= ctx + jq;
                z[v] = vis ? s[v] * p.score_mul : -INFINITY;
                mx = fmaxf(mx, z[v]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float mn = fmaxf(run_m, mx);
            const float m_use = mn == -INFINITY ? 0.f : mn;
            const float alpha = exp2f(run_m - m_use);
            run_m = mn;
            run_l *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
            float pr[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                pr[v] = exp2f(z[v] - m_use);
                run_l += pr[v];
            }
            // ---- O^T += V^T P^T; K step ks covers the lane's accumulator values v = 8 ks .. 8 ks + 7,
            // i.e. keys 16 ks + 8 (e/4) + 4 hi + e%4 for slot e
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pf = pack8(pr + 8 * ks);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint16_t *vrow = &sV[(32 * mb + col) * SVS + 16 * ks + 4 * hi];
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                    const uint2 up = *reinterpret_cast<const uint2 *>(vrow + 8);
                    const uint4 raw = {lo.x, lo.y, up.x, up.y};
                    acc[mb] = mma32(__builtin_bit_cast(bf16x8, raw), pf, acc[mb]);
                }
            }
        }
        __syncthreads();
    }

    run_l += __shfl_xor(run_l, 32, kWave);
    if (jq < p.chunk) {
        const float inv = p.out_mul / run_l;
        float *o = out + (int64_t(jq) * p.h + head) * p.d_h;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int d = 32 * mb + 8 * (v >> 2) + 4 * hi + (v & 3);
                if (d < p.d_h) o[d] = acc[mb][v] * inv;
            }
    }
}

template <int HP, int DP, int RH>
hipError_t launch_one(const PrefillParams &p, hipStream_t s) {
    const dim3 grid((p.chunk + kQT - 1) / kQT, p.h, p.batch);
    hipLaunchKernelGGL((prefill_kernel<HP, DP, RH>), grid, dim3(kPrefillThreads), 0, s, p);
    return hipGetLastError();
}

template <int HP, int DP>
hipError_t launch_rank(int RH, const PrefillParams &p, hipStream_t s) {
    switch (RH) {
        case 1: return launch_one<HP, DP, 1>(p, s);
        case 2: return launch_one<HP, DP, 2>(p, s);
        case 4: return launch_one<HP, DP, 4>(p, s);
    }
    return hipErrorInvalidValue;
}

#define TPA_PREFILL_SHAPES(X) X(16, 64) X(16, 128) X(32, 64) X(32, 128) X(64, 64) X(64, 128)

}  // namespace

bool prefill_supported(const Layout &L) {
    if (L.es != 2) return false;
#define X(HP_, DP_) \
    if (L.HP == HP_ && L.DP == DP_) return true;
    TPA_PREFILL_SHAPES(X)
#undef X
    return false;
}

hipError_t launch_prefill(const Layout &L, const PrefillParams &p, hipStream_t s) {
#define X(HP_, DP_) \
    if (L.es == 2 && L.HP == HP_ && L.DP == DP_) return launch_rank<HP_, DP_>(L.RH, p, s);
    TPA_PREFILL_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tpa
