// Causal chunked prefill over a TPA factor cache.
//
// TPA notes page, Key design: K_s = (1/R_K) A_K[s]^T B_K[s] and V_s likewise;
// FlashTPA: no full K/V in device memory.  A prefill chunk has many query
// rows per head, so each work-group rebuilds one head's key and value rows of
// a 64-token tile on chip,
//     K~_i[s,:] = sum_r A_K[s,r,i] B~_K[s,r,:]      (1/R_K folded into the scale)
//     V_i[s,:]  = sum_r A_V[s,r,i] B_V[s,r,:]       (1/R_V applied at the end)
// in fp32 from the cached factors, rounds them once to bf16 into LDS, and
// runs a flash-attention loop on the bf16 matrix cores (32x32x16):
//     S^T = K~_i Q~^T   (M = keys, N = queries, K = d_h)
//     causal mask: chunk row j (position ctx + j) sees keys 0 .. ctx + j
//     online softmax per query (a lane owns one query column)
//     O^T += V_i^T P^T  (M = d_h, N = queries, K = keys)
// A work-group owns 256 query rows of one head (8 waves x 32), so every
// (key, head) pair is rebuilt at most twice per chunk of 512 rows.  The LDS
// tiles are double-buffered: the waves rebuild tile t+1 while their matrix
// cores work on tile t.  The key order inside the value contraction is
// permuted (bits 2 and 3 of the key index swapped within each group of 16)
// so that the score accumulator a lane holds is exactly its slice of P^T and
// its slice of V^T is one 16-byte LDS read.
#include "common.h"

namespace tpa {
namespace {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kQT = 32 * kPrefillWaves;  // query rows per work-group
constexpr int kKT = 64;                  // keys per tile

__device__ __forceinline__ floatx16 mma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return uint32_t(f32_to_bf16_rne(a)) | (uint32_t(f32_to_bf16_rne(b)) << 16);
}

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    const uint4 v = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void unpack8(uint4 raw, float *x) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
}

__device__ __forceinline__ void unpack4(uint2 raw, float *x) {
    x[0] = __uint_as_float(raw.x << 16);
    x[1] = __uint_as_float(raw.x & 0xffff0000u);
    x[2] = __uint_as_float(raw.y << 16);
    x[3] = __uint_as_float(raw.y & 0xffff0000u);
}

// LDS position of tile key k inside the value contraction's key order
__device__ __forceinline__ int vpos(int k) { return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3); }

template <int HP, int DP, int RH>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
    constexpr int KS = DP / 16;  // score K steps
    constexpr int MB = DP / 32;  // value M blocks
    constexpr int NB = HP / 16;
    constexpr int KBS = DP / 32;  // B~_K 32-wide column blocks in the cache layout
    constexpr int MBV = DP / 16;
    constexpr int TOK = kRows / RH;
    constexpr int SKS = DP + 8;   // LDS row stride of K~ (bf16 elements)
    constexpr int SVS = kKT + 8;  // LDS row stride of V^T
    constexpr int64_t BLK = 2LL * kRows * (HP + DP);
    constexpr int OFF_AV = kRows * HP, OFF_BK = 2 * kRows * HP, OFF_BV = 2 * kRows * HP + kRows * DP;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKT * SKS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][DP * SVS];

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
    const int j_last = min(p.chunk, j0 + kQT) - 1;
    const int n_keys = ctx + j_last + 1;  // keys any row of this work-group sees (all appended)
    const int n_kt = (n_keys + kKT - 1) / kKT;
    const int gate_lane = head & 15, gate_nb = head >> 4;

    // ---- rebuild K~_i and V_i^T of tile kt into LDS buffer `buf`
    auto rebuild = [&](int kt, int buf) {
        const int key0 = kt * kKT;
        uint16_t *dK = sK[buf];
        uint16_t *dV = sV[buf];
        // K~ rows: item = (key, 8 features)
        for (int it = tid; it < kKT * (DP / 8); it += kPrefillThreads) {
            const int k = it / (DP / 8), c8 = it % (DP / 8);
            const int key = key0 + k;
            float kv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[e] = 0.f;
            if (key < n_keys) {
                const uint16_t *blk = seq + int64_t(key / TOK) * BLK;
                const int row0 = (key % TOK) * RH;
                const int mb = row0 >> 4, g4 = (row0 & 15) >> 2, v0 = row0 & 3;
                float a[4];
                unpack4(*reinterpret_cast<const uint2 *>(blk + ((mb * NB + gate_nb) * kWave + 16 * g4 + gate_lane) * 4),
                        a);
                const int d0 = 8 * c8, kb = d0 >> 5, lsub = (d0 & 31) >> 3;
#pragma unroll
                for (int r = 0; r < RH; ++r) {
                    const int row = row0 + r;
                    float bk[8];
                    unpack8(*reinterpret_cast<const uint4 *>(
                                blk + OFF_BK + (((row >> 4) * KBS + kb) * kWave + 16 * lsub + (row & 15)) * 8),
                            bk);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] += a[v0 + r] * bk[e];
                }
            }
            *reinterpret_cast<bf16x8 *>(&dK[k * SKS + 8 * c8]) = pack8(kv);
        }
        // V^T columns: item = (block of the tile, 16-feature group, lane of the cache chunk); the
        // 16-byte chunk holds 8 factor rows (whole tokens) of one feature
        constexpr int BPT = kKT / TOK;  // cache blocks per tile
        for (int it = tid; it < BPT * MBV * kWave; it += kPrefillThreads) {
            const int bi = it / (MBV * kWave), rem = it % (MBV * kWave);
            const int mv = rem / kWave, cl = rem % kWave;
            const int g4 = cl >> 4, d = 16 * mv + (cl & 15);
            const int kbase = bi * TOK;  // tile-relative key of the block's first token
            const bool live = key0 + kbase < n_keys;
            float x[8], ga[2][4];
            if (live) {
                const uint16_t *blk = seq + int64_t((key0 + kbase) / TOK) * BLK;
                unpack8(*reinterpret_cast<const uint4 *>(blk + OFF_BV + (mv * kWave + cl) * 8), x);
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    unpack4(*reinterpret_cast<const uint2 *>(
                                blk + OFF_AV + ((m * NB + gate_nb) * kWave + 16 * g4 + gate_lane) * 4),
                            ga[m]);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                // rows 16 m + 4 g4 + 0..3 of the block: 4 / RH whole tokens
                constexpr int TPH = 4 / RH;
                float vt[TPH];
#pragma unroll
                for (int tl = 0; tl < TPH; ++tl) {
                    float acc = 0.f;
                    if (live) {
#pragma unroll
                        for (int r = 0; r < RH; ++r) acc += ga[m][tl * RH + r] * x[4 * m + tl * RH + r];
                    }
                    const int key = kbase + (16 * m + 4 * g4) / RH + tl;
                    vt[tl] = key0 + key < n_keys ? acc : 0.f;
                }
                const int k0 = kbase + (16 * m + 4 * g4) / RH;
                uint16_t *dst = &dV[d * SVS + vpos(k0)];
                if (TPH == 4) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2(vt[0], vt[TPH > 1 ? 1 : 0]),
                                                                 pack2(vt[TPH > 2 ? 2 : 0], vt[TPH > 3 ? 3 : 0]));
                } else if (TPH == 2) {
                    *reinterpret_cast<uint32_t *>(dst) = pack2(vt[0], vt[TPH > 1 ? 1 : 0]);
                } else {
                    *dst = f32_to_bf16_rne(vt[0]);
                }
            }
        }
    };

    // Q operand (B of S^T): lane supplies Q~[jq][16 ks + 8 hi + e]
    bf16x8 qf[KS];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) + (int64_t(b) * p.chunk + jq) * p.h * p.d_h +
                               int64_t(head) * p.d_h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * hi;
            if (jq < p.chunk && d0 < p.d_h && (p.d_h & 7) == 0) {
                qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + d0));
            } else {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (jq < p.chunk && d0 + e < p.d_h) ? bf16_to_f32(qrow[d0 + e]) : 0.f;
                qf[ks] = pack8(x);
            }
        }
    }

    floatx16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][v] = 0.f;
    float run_m = -INFINITY, run_l = 0.f;
    const int wave_last = min(p.chunk - 1, jw + 31);

    rebuild(0, 0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < n_kt) rebuild(kt + 1, buf ^ 1);
        const int key0 = kt * kKT;
        if (jw < p.chunk && key0 <= ctx + wave_last) {
            const uint16_t *cK = sK[buf];
            const uint16_t *cV = sV[buf];
            // ---- S^T = K~ Q~^T for two 32-key blocks
            floatx16 s[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
                for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cK[(32 * kb2 + col) * SKS + 16 * ks + 8 * hi]);
                    s[kb2] = mma32(a, qf[ks], s[kb2]);
                }
            }
            // ---- causal mask, online softmax (log2 units)
            float mx = -INFINITY;
            const bool full = key0 + kKT - 1 <= ctx + jw;  // no key of the tile is beyond any row of the wave
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = key0 + 32 * kb2 + 8 * (v >> 2) + 4 * hi + (v & 3);
                    const bool vis = jq < p.chunk && (full || key <= ctx + jq);
                    s[kb2][v] = vis ? s[kb2][v] * p.score_mul : -INFINITY;
                    mx = fmaxf(mx, s[kb2][v]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float mn = fmaxf(run_m, mx);
            const float m_use = mn == -INFINITY ? 0.f : mn;
            const float alpha = exp2f(run_m - m_use);
            run_m = mn;
            run_l *= alpha;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    s[kb2][v] = exp2f(s[kb2][v] - m_use);
                    run_l += s[kb2][v];
                }
            // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
            for (int ks4 = 0; ks4 < 4; ++ks4) {
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = s[ks4 >> 1][8 * (ks4 & 1) + e];
                const bf16x8 pf = pack8(x);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cV[(32 * mb + col) * SVS + 16 * ks4 + 8 * hi]);
                    acc[mb] = mma32(a, pf, acc[mb]);
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
            for (int v4 = 0; v4 < 4; ++v4) {
                const int d = 32 * mb + 8 * v4 + 4 * hi;
                if (d + 3 < p.d_h && (p.d_h & 3) == 0) {
                    *reinterpret_cast<float4 *>(o + d) = make_float4(acc[mb][4 * v4] * inv, acc[mb][4 * v4 + 1] * inv,
                                                                     acc[mb][4 * v4 + 2] * inv, acc[mb][4 * v4 + 3] * inv);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (d + u < p.d_h) o[d + u] = acc[mb][4 * v4 + u] * inv;
                }
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
