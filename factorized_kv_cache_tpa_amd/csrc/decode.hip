// Split-sequence decode over a TPA factor cache.
//
// TPA notes page, Key design: K_s = (1/R_K) A_K[s]^T B_K[s] and V_s likewise;
// FlashTPA: attention is evaluated from the factors, never from a built K/V.
// For one query row q~ (already rotated) and head i:
//   z_s,i = scale * q~_i . K~_s[i,:] = (scale/R_K) sum_r A_K[s,r,i] (B~_K[s,r,:] . q~_i)
//   out_i = sum_s softmax_s(z_s,i) V_s[i,:]
//         = (1/R_V) sum_s sum_r (p_s,i A_V[s,r,i]) B_V[s,r,:] / sum_s p_s,i
// Both inner sums are matrix-core contractions with the heads as the N
// dimension:
//   1. U^T[(s,r), i] = B~_K[(s,r), :] . q~^T[:, i]   (M = token rows, K = d_h)
//   2. gate: z[s, i] = sum_r A_K[s,r,i] U^T[(s,r), i]  (in-lane: a lane's four
//      accumulator rows hold whole tokens because the padded rank is 1, 2 or 4)
//   3. online softmax per head (running max in log2 units, running sum)
//   4. W[(s,r), i] = p[s,i] A_V[s,r,i], rounded once to the element type (at
//      rank 1 with bf16 operands: as a pair hi + lo, see kSplitW)
//   5. O^T[:, i] += B_V[(s,r), :]^T W[(s,r), i]     (M = d_h, K = token rows)
// The cache block layout (common.h) makes the score accumulator of a lane
// exactly the k-slice it feeds to step 5, so no data crosses lanes between
// the contractions.  The batch's blocks are shared out evenly over the
// work-groups (4 waves each), which therefore cover pieces of one or more
// sequences whatever their lengths; for each piece the waves take interleaved
// blocks, merge in LDS and write one partial (max, sum, unnormalized output);
// a second kernel merges the pieces of each sequence:
//   M = max_j m_j,  out = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j.
// (Fixed-size splits per sequence left a ragged batch's long sequences running
// alone at the end: 74% of HBM peak where equal lengths of the same total
// reach 87%.)
// (Merging in the same launch by the last work-group to finish a sequence was
// measured slower on MI355X: the agent-scope release / acquire every
// work-group then needs writes back and invalidates its XCD's L2.)
#include <climits>
#include <type_traits>

#include "common.h"

namespace tpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLazy = 8.0f;  // headroom of the lazy reference max, log2 units (weights <= 256)

template <typename T>
struct Mfma;

template <>
struct Mfma<uint16_t> {  // bf16 in, fp32 accumulate: v_mfma_f32_16x16x32_bf16
    static constexpr int E = 8;
    typedef bf16x8 Frag;
    __device__ static Frag load(const uint16_t *p) { return __builtin_bit_cast(Frag, *reinterpret_cast<const uint4 *>(p)); }
    __device__ static Frag stream(const uint16_t *p) { return __builtin_bit_cast(Frag, stream_load16(p)); }
    __device__ static Frag pack(const float *x) {
        const uint4 v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                   pack_bf16x2(x[6], x[7]));
        return __builtin_bit_cast(Frag, v);
    }
    // zero the slots whose flag bit is set
    __device__ static Frag mask(Frag f, unsigned zero_bits) {
        uint4 v = __builtin_bit_cast(uint4, f);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (zero_bits & (1u << e)) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        v.x = w[0];
        v.y = w[1];
        v.z = w[2];
        v.w = w[3];
        return __builtin_bit_cast(Frag, v);
    }
    typedef u32x2 GateRaw;  // four bf16 gates
    __device__ static GateRaw load_gates(const uint16_t *p) { return stream_load8(p); }
    __device__ static void unpack_gates(GateRaw v, float *g) {
        g[0] = __uint_as_float(v.x << 16);
        g[1] = __uint_as_float(v.x & 0xffff0000u);
        g[2] = __uint_as_float(v.y << 16);
        g[3] = __uint_as_float(v.y & 0xffff0000u);
    }
    // q~[head][d0 .. d0+7]; zeros outside h x d_h (d_h even, so a chunk of 8 is all in or all out
    // when d_h % 8 == 0; otherwise element by element)
    __device__ static Frag load_q(const uint16_t *qb, int head, int d0, int h, int d_h) {
        if (head >= h || d0 >= d_h) return __builtin_bit_cast(Frag, make_uint4(0, 0, 0, 0));
        const uint16_t *src = qb + int64_t(head) * d_h + d0;
        if ((d_h & 7) == 0) return load(src);
        float x[8];
        for (int e = 0; e < 8; ++e) x[e] = d0 + e < d_h ? bf16_to_f32(src[e]) : 0.f;
        return pack(x);
    }
    __device__ static float value(Frag f, int e) {
        const uint4 v = __builtin_bit_cast(uint4, f);
        const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    // RoPE of a loaded fragment q[head][d0 .. d0+7] (d0 even: four whole pairs), cs = cos/sin table
    __device__ static Frag rotate_q(Frag f, int d0, const float *cs) {
        const uint4 v = __builtin_bit_cast(uint4, f);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = (d0 >> 1) + k;
            float y0, y1;
            rope_rotate(bf16_to_f32(uint16_t(w[k] & 0xffffu)), bf16_to_f32(uint16_t(w[k] >> 16)), cs[2 * j],
                        cs[2 * j + 1], y0, y1);
            o[k] = pack_bf16x2(y0, y1);
        }
        return __builtin_bit_cast(Frag, make_uint4(o[0], o[1], o[2], o[3]));
    }
    __device__ static floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<float> {  // fp32 in, fp32 accumulate: v_mfma_f32_16x16x4_f32
    static constexpr int E = 1;
    typedef float Frag;
    __device__ static Frag load(const float *p) { return *p; }
    __device__ static Frag stream(const float *p) { return __builtin_nontemporal_load(p); }
    __device__ static Frag pack(const float *x) { return x[0]; }
    __device__ static Frag mask(Frag f, unsigned zero_bits) { return (zero_bits & 1u) ? 0.0f : f; }
    typedef u32x4 GateRaw;
    __device__ static GateRaw load_gates(const float *p) { return stream_load16(p); }
    __device__ static void unpack_gates(GateRaw v, float *g) {
        g[0] = __uint_as_float(v.x);
        g[1] = __uint_as_float(v.y);
        g[2] = __uint_as_float(v.z);
        g[3] = __uint_as_float(v.w);
    }
    __device__ static Frag load_q(const float *qb, int head, int d0, int h, int d_h) {
        return (head < h && d0 < d_h) ? qb[int64_t(head) * d_h + d0] : 0.f;
    }
    __device__ static float value(Frag f, int) { return f; }
    // RoPE of q[head][d0]: its pair partner d0 ^ 1 sits in the lane 16 apart (g ^ 1, same head)
    __device__ static Frag rotate_q(Frag f, int d0, const double *cs) {
        const float partner = __shfl_xor(f, 16, kWave);
        const int j = d0 >> 1;
        const double a = (d0 & 1) ? partner : f, b = (d0 & 1) ? f : partner;
        double y0, y1;
        rope_rotate(a, b, cs[2 * j], cs[2 * j + 1], y0, y1);
        return float((d0 & 1) ? y1 : y0);
    }
    __device__ static floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float wave_max_across_groups(float x) {
    // lanes l, l^16, l^32, l^48 hold the same head
    x = fmaxf(x, __shfl_xor(x, 16, kWave));
    x = fmaxf(x, __shfl_xor(x, 32, kWave));
    return x;
}

__device__ __forceinline__ float wave_sum_across_groups(float x) {
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// Query modes, each its own instantiation so the plain decode carries none of the others:
//   kQRot  -- q arrives rotated (tpa_decode);
//   kStep  -- a fused step: q arrives unrotated, the sequence's first job carries the new token (tpa_decode_step);
//   kQFact -- q arrives as factors A_Q, B_Q (unrotated), q~ = RoPE((1/R_Q) A_Q^T B_Q) at position len
//             (tpa_decode_fq).
constexpr int kQRot = 0, kStepMode = 1, kQFact = 2;
constexpr int kMaxRQ = 16;  // query rank limit of the factored mode

// kF8: the cache holds E4M3 codes in the paired 8-bit layout (T = uint16_t: bf16 queries and operands).
template <typename T, int HP, int DP, int RH, int kMode, bool kF8>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
    static_assert(!kF8 || (sizeof(T) == 2 && (DP / 16) % 2 == 0), "E4M3 storage: bf16 operands, paired value blocks");
    constexpr bool kStep = kMode == kStepMode;
    constexpr bool kFact = kMode == kQFact;
    using M = Mfma<T>;
    using Frag = typename M::Frag;
    using GateRaw = typename M::GateRaw;
    constexpr int E = M::E;
    constexpr int NB = HP / 16;           // head blocks (MFMA N)
    constexpr int KBS = DP / (4 * E);     // score K blocks
    constexpr int MBV = DP / 16;          // value M blocks
    constexpr int KBV = kRows / (4 * E);  // value K blocks
    constexpr int TOK = kRows / RH;       // tokens per cache block
    constexpr int TPL = 4 / RH;           // tokens per lane per score row block
    // Rank 1 with bf16 operands: each token's value row carries its whole weight p A_V, so the weights go
    // to the matrix cores as a bf16 pair hi + lo (two products with the same B_V operand; the matrix cores
    // have slack in this memory-bound loop), which leaves the weights exact to ~2^-17.
    constexpr bool kSplitW = RH == 1 && sizeof(T) == 2;
    constexpr int64_t BLK = 2LL * kRows * (HP + DP);
    constexpr int OFF_AV = kRows * HP, OFF_BK = 2 * kRows * HP, OFF_BV = 2 * kRows * HP + kRows * DP;

    using F = typename RopeMath<T>::F;
    // per-wave (max, sum); row kWaves holds a fused step's new token (first job), else (-inf, 0)
    __shared__ float sm_m[kWaves + 1][HP];
    __shared__ float sm_l[kWaves + 1][HP];
    __shared__ __attribute__((aligned(16))) float sm_o[kWaves][HP][DP + 4];
    constexpr int SH = kStep ? HP : 1, SD = (kStep || kFact) ? DP : 2;
    // factored query: A_Q, B~_Q staged as fp32, then q~ built once per work-group (element type)
    constexpr int QR = kFact ? kMaxRQ : 1, QH = kFact ? HP : 4, QD = kFact ? DP : 4;
    __shared__ __attribute__((aligned(16))) float sm_aq[QR][QH];
    __shared__ __attribute__((aligned(16))) float sm_bq[QR][QD];
    __shared__ __attribute__((aligned(16))) T sm_q[QH][QD + 8];
    __shared__ F sm_cs[SD];             // fused step, factored query: cos/sin of the query's position
    __shared__ float sm_na[2][RH][SH];  // fused step, first job: the new token's A_K, A_V
    __shared__ __attribute__((aligned(16))) float sm_nb[2][RH][SD];  // ... its B_K, B_V (unrotated)
    __shared__ float sm_wt[SH];         // ... and the weight of its value row per head (in-group merge)
    static_assert(RH * HP <= kThreads && RH * DP / 2 <= kThreads && DP / 2 <= kThreads,
                  "one new-token item and one RoPE pair per thread");

    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform: scalar addressing
    const int g = lane >> 4, c = lane & 15;
    const int tid = threadIdx.x;

    // ---- Work partition.  Sequence b owns v_b = max(ceil(len_b / TOK), 1) virtual blocks (1 if it is
    // rejected), laid end to end in batch order; work-group wg takes the virtual blocks [wg P, (wg + 1) P)
    // (P = per_wg)
    // and runs one job per sequence that range touches: that piece of the sequence's blocks, folded into
    // one partial at index wg + b (along the partition (wg, b) only ever steps up, in one or both, so the
    // index is unique).  The blocks are shared out evenly however ragged the lengths, and every work-group
    // finds its range from the lengths itself (no planning launch).
    struct SeqInfo {
        int len, vb;
        int64_t start;
        bool rejected;
    };
    auto seq_info = [&](int bb) -> SeqInfo {
        SeqInfo si;
        const int ln = p.seq_len[bb];
        si.len = ln < 0 ? 0 : (ln > p.max_len ? p.max_len : ln);
        si.start = p.seq_start[bb];
        // A sequence that is misaligned, or whose slots (a fused step: and the new token's slot) reach past
        // the capacity, is not read at all: NaN output.
        si.rejected = seq_rejected(si.start, int64_t(si.len) + (kStep ? 1 : 0), TOK, p.capacity);
        si.vb = si.rejected ? 1 : max((si.len + TOK - 1) / TOK, 1);
        return si;
    };
    __shared__ int sm_wsum[kWaves];
    __shared__ int sm_wmin[kWaves], sm_wmax[kWaves];
    __shared__ int sm_first[2];  // the first sequence of this work-group's range, and its first virtual block
    __shared__ int64_t sm_first_start;  // ... and that sequence's start, length, virtual blocks, state
    __shared__ int sm_first_len, sm_first_vb, sm_first_rej;
    const int wg = blockIdx.x;
    const int per = (p.batch + kThreads - 1) / kThreads;  // sequences per thread in the scan
    const int b_lo = min(p.batch, tid * per), b_hi = min(p.batch, b_lo + per);
    int mine = 0;  // (the host bounds the batch's virtual blocks below 2^31)
    int vmin = INT_MAX, vmax = 0;
    SeqInfo lo_si{0, 0, 0, false};  // the thread's first sequence, kept (one sequence per thread up to 256)
    for (int bb = b_lo; bb < b_hi; ++bb) {
        const SeqInfo si = seq_info(bb);
        if (bb == b_lo) lo_si = si;
        mine += si.vb;
        vmin = min(vmin, si.vb);
        vmax = max(vmax, si.vb);
    }
    int incl = mine;  // inclusive scan over the wave, then over the waves through LDS
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
        vmin = min(vmin, __shfl_xor(vmin, o, kWave));
        vmax = max(vmax, __shfl_xor(vmax, o, kWave));
    }
    if (lane == kWave - 1) sm_wsum[w] = incl;
    if (lane == 0) {
        sm_wmin[w] = vmin;
        sm_wmax[w] = vmax;
    }
    __syncthreads();
    int excl = incl - mine, V = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
        excl += ww < w ? sm_wsum[ww] : 0;
        V += sm_wsum[ww];
        vmin = min(vmin, sm_wmin[ww]);
        vmax = max(vmax, sm_wmax[ww]);
    }
    V = __builtin_amdgcn_readfirstlane(V);  // the same in every lane: scalar registers
    vmax = __builtin_amdgcn_readfirstlane(vmax);
    // Blocks per work-group: the caller's, or the batch's share of the grid.  When every sequence has the
    // same number of blocks (and the grid has a work-group for each), each is cut into k equal pieces
    // instead, k work-groups per sequence and none straddling two sequences (for short pieces a second job
    // costs more than the imbalance it removes): the same partition with every sequence padded to k pieces.
    int per_wg = p.split_blocks, stride = 0;  // stride: virtual blocks per sequence when padded
    if (per_wg <= 0) {
        auto round_up = [&](int x) {
            x = (x + kWaves - 1) / kWaves * kWaves;
            // a short piece (two blocks per wave or fewer) is latency-bound: fewer, longer pieces halve
            // the partials to merge and cost no bandwidth
            return x <= 2 * kWaves ? 4 * kWaves : x;
        };
        if (__builtin_amdgcn_readfirstlane(vmin) == vmax && int64_t(gridDim.x) >= p.batch) {
            const int k0 = max(1, int(gridDim.x) / p.batch);
            per_wg = round_up((vmax + k0 - 1) / k0);
            stride = (vmax + per_wg - 1) / per_wg * per_wg;
            V = stride * p.batch;
        } else {
            per_wg = round_up((V + int(gridDim.x) - 1) / int(gridDim.x));
        }
    }
    per_wg = __builtin_amdgcn_readfirstlane(per_wg);
    stride = __builtin_amdgcn_readfirstlane(stride);
    const int gs = wg * per_wg;
    if (gs >= V) return;  // nothing left for this work-group (uniform)
    const int ge = __builtin_amdgcn_readfirstlane(min(V, gs + per_wg));
    if (stride > 0) {  // padded: the first sequence is gs / stride
        const int b0 = gs / stride;
        if (b0 >= b_lo && b0 < b_hi) {
            const SeqInfo si = b0 == b_lo ? lo_si : seq_info(b0);
            sm_first[0] = b0;
            sm_first[1] = b0 * stride;
            sm_first_start = si.start;
            sm_first_len = si.len;
            sm_first_vb = si.vb;
            sm_first_rej = si.rejected;
        }
    } else if (gs >= excl && gs < excl + mine) {  // the one thread whose sequences hold virtual block gs
        int bb = b_lo;
        SeqInfo si = lo_si;
        while (gs >= excl + si.vb) {  // (only with more than one sequence per thread)
            excl += si.vb;
            si = seq_info(++bb);
        }
        sm_first[0] = bb;
        sm_first[1] = excl;
        sm_first_start = si.start;
        sm_first_len = si.len;
        sm_first_vb = si.vb;
        sm_first_rej = si.rejected;
    }
    __syncthreads();

    // One job: blocks [blk_begin, blk_end_v) of sequence b (virtual blocks past its last real one hold
    // nothing), its partial at index part.  first: the job holds the sequence's first block, last: its last.
    auto run_job = [&](const int b, const SeqInfo si, const int64_t part, const int blk_begin, const int blk_end_v,
                       const bool first_job, const bool last_job) {
        // lane and wave indices through opaque copies, so that nothing derived from them is hoisted out of the
        // job loop and held across the whole job (the body was written as straight-line code)
        int lane_o = lane, tid_o = tid, w_o = w;
        asm volatile("" : "+v"(lane_o), "+v"(tid_o), "+s"(w_o));
        const int lane = lane_o, tid = tid_o, w = w_o;
        const int g = lane >> 4, c = lane & 15;
        const int len = si.len;
        const int64_t start = si.start;
        const bool rejected = si.rejected;
        const int nblk = (len + TOK - 1) / TOK;
        // A fused step's first job carries the step's new token (even over an empty sequence): it folds the
        // token's own score and value into its partial ...
        const bool new_tok = kStep && first_job && !rejected;
        // ... and its last job writes the token's record (for a long sequence the two land on different
        // work-groups)
        const bool rec_tok = kStep && last_job && !rejected;
        if (rejected || (blk_begin >= nblk && !new_tok)) {
            // A job with no tokens (an empty or rejected sequence) marks its partial empty (max -inf, sum 0);
            // the merge writes zeros (empty) or NaN (rejected).
            for (int head = threadIdx.x; head < HP; head += kThreads)
                *reinterpret_cast<float2 *>(p.ws_ml + (part * HP + head) * 2) = make_float2(-INFINITY, 0.f);
            return;
        }
        const int blk_end = min(nblk, blk_end_v);
        const int full_end = min(blk_end, len / TOK);  // blocks [blk_begin, full_end) hold TOK valid tokens
        constexpr int CES = kF8 ? 1 : int(sizeof(T));  // bytes per stored element
        const char *seq = reinterpret_cast<const char *>(p.cache) + (start / TOK) * BLK * CES;

        // One block's operands, loaded straight from the cache in MFMA lane order: a scalar block base
        // plus one per-lane offset, so every load is one instruction with an immediate region offset.
        struct StageNative {
            GateRaw ak[2][NB], av[2][NB];
            Frag bk[2][KBS], bv[MBV][KBV];
        };
        // E4M3: a lane's 16 bytes hold its codes for both row blocks of a k-block (B~_K) or for value blocks
        // 2j and 2j+1 (B_V); its 8 gate bytes hold both row blocks of a head block.  Decoded at use.
        struct StageF8 {
            u32x2 ak[NB], av[NB];
            u32x4 bk[KBS], bv[MBV / 2];
        };
        using Stage = std::conditional_t<kF8, StageF8, StageNative>;
        const uint32_t off_op = uint32_t(lane * E * sizeof(T));  // operand lane offset, bytes (native)
        const uint32_t off_gt = uint32_t(lane * 4 * sizeof(T));  // gate lane offset, bytes (native)
        auto load = [&](Stage &st, int blk, bool real = true) {
            const char *bp = real ? seq + int64_t(blk) * BLK * CES : reinterpret_cast<const char *>(p.cache);
            if constexpr (kF8) {
                const char *op = bp + lane * 16;
                const char *gt = bp + lane * 8;
#pragma unroll
                for (int kb = 0; kb < KBS; ++kb) st.bk[kb] = stream_load16(op + OFF_BK + kb * kWave * 16);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    st.ak[nb] = stream_load8(gt + nb * kWave * 8);
                    st.av[nb] = stream_load8(gt + OFF_AV + nb * kWave * 8);
                }
#pragma unroll
                for (int j = 0; j < MBV / 2; ++j) st.bv[j] = stream_load16(op + OFF_BV + j * kWave * 16);
            } else {
                const T *op = reinterpret_cast<const T *>(bp + off_op);
                const T *gt = reinterpret_cast<const T *>(bp + off_gt);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int kb = 0; kb < KBS; ++kb)
                        st.bk[mb][kb] = M::stream(op + OFF_BK + (mb * KBS + kb) * kWave * E);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        st.ak[mb][nb] = M::load_gates(gt + (mb * NB + nb) * kWave * 4);
                        st.av[mb][nb] = M::load_gates(gt + OFF_AV + (mb * NB + nb) * kWave * 4);
                    }
#pragma unroll
                for (int mv = 0; mv < MBV; ++mv)
#pragma unroll
                    for (int q = 0; q < KBV; ++q) st.bv[mv][q] = M::stream(op + OFF_BV + (mv * KBV + q) * kWave * E);
            }
        };
        // The operands of a loaded stage: B~_K fragment (row block mb, k-block kb), the 4 gates of row block
        // mb and head block nb, and the B_V fragment of value block mv (k-block q).
        auto frag_bk = [&](const Stage &st, int mb, int kb) -> Frag {
            if constexpr (kF8) {
                const u32x4 r = st.bk[kb];
                return __builtin_bit_cast(Frag, mb ? e4m3x8_to_bf16x8(r.z, r.w) : e4m3x8_to_bf16x8(r.x, r.y));
            } else {
                return st.bk[mb][kb];
            }
        };
        auto gates = [&](const Stage &st, bool value, int mb, int nb, float *gv) {
            if constexpr (kF8) {
                const u32x2 r = value ? st.av[nb] : st.ak[nb];
                e4m3x4_to_f32(mb ? r.y : r.x, gv);
            } else {
                M::unpack_gates(value ? st.av[mb][nb] : st.ak[mb][nb], gv);
            }
        };
        auto frag_bv = [&](const Stage &st, int mv, int q) -> Frag {
            if constexpr (kF8) {
                const u32x4 r = st.bv[mv >> 1];
                return __builtin_bit_cast(Frag, (mv & 1) ? e4m3x8_to_bf16x8(r.z, r.w) : e4m3x8_to_bf16x8(r.x, r.y));
            } else {
                return st.bv[mv][q];
            }
        };

        // Fused step, first job: this thread's item of the new token (one head-factor pair (A_K, A_V) of row
        // r, head i, and one feature pair (d, d+1) of B_K and B_V of row r), loaded before everything else:
        // memory returns in order, so these must not queue behind the factor stream.
        const int na_r = tid / HP, na_i = tid % HP, nb_r = tid / (DP / 2), nb_d = 2 * (tid % (DP / 2));
        T nak = T(0), nav = T(0), nbk0 = T(0), nbk1 = T(0), nbv0 = T(0), nbv1 = T(0);
        if (kStep && (new_tok || rec_tok)) {
            const T *AK = reinterpret_cast<const T *>(p.st.A_K) + int64_t(b) * p.RK * p.h;
            const T *AV = reinterpret_cast<const T *>(p.st.A_V) + int64_t(b) * p.RV * p.h;
            const T *BK = reinterpret_cast<const T *>(p.st.B_K) + int64_t(b) * p.RK * p.d_h;
            const T *BV = reinterpret_cast<const T *>(p.st.B_V) + int64_t(b) * p.RV * p.d_h;
            if (na_r < p.RK && na_i < p.h) nak = AK[na_r * p.h + na_i];
            if (na_r < p.RV && na_i < p.h) nav = AV[na_r * p.h + na_i];
            if (nb_r < p.RK && nb_d < p.d_h) {
                nbk0 = BK[nb_r * p.d_h + nb_d];
                nbk1 = BK[nb_r * p.d_h + nb_d + 1];
            }
            if (nb_r < p.RV && nb_d < p.d_h) {
                nbv0 = BV[nb_r * p.d_h + nb_d];
                nbv1 = BV[nb_r * p.d_h + nb_d + 1];
            }
        }
        for (int head = tid; head < HP; head += kThreads) {
            sm_m[kWaves][head] = -INFINITY;
            sm_l[kWaves][head] = 0.f;
        }
        // fused step, factored query: this thread's RoPE frequency (pair j = tid), read now for the same reason
        const double theta_j = (kStep || kFact) && tid < DP / 2 ? p.rope.theta[tid] : 0.0;

        // Factored query: this thread's share of A_Q (row-major [R_Q][h]) and B_Q ([R_Q][d_h], unrotated),
        // loaded before the stream for the same reason; elements past the real sizes are zeros.
        constexpr int QA_PER = kFact ? (kMaxRQ * HP + kThreads - 1) / kThreads : 1;
        constexpr int QB_PER = kFact ? (kMaxRQ * DP + kThreads - 1) / kThreads : 1;
        float qa_raw[QA_PER], qb_raw[QB_PER];
        if constexpr (kFact) {
            const T *AQ = reinterpret_cast<const T *>(p.a_q) + int64_t(b) * p.r_q * p.h;
            const T *BQ = reinterpret_cast<const T *>(p.q) + int64_t(b) * p.r_q * p.d_h;
#pragma unroll
            for (int k = 0; k < QA_PER; ++k) {
                const int idx = tid + k * kThreads, r = idx / HP, i = idx % HP;
                qa_raw[k] = r < p.r_q && i < p.h ? Elem<T>::to_f32(AQ[r * p.h + i]) : 0.f;
            }
#pragma unroll
            for (int k = 0; k < QB_PER; ++k) {
                const int idx = tid + k * kThreads, r = idx / DP, d = idx % DP;
                qb_raw[k] = r < p.r_q && d < p.d_h ? Elem<T>::to_f32(BQ[r * p.d_h + d]) : 0.f;
            }
        }

        // query operand (B of the score contraction; loaded first: memory returns in order, so the first
        // block can start as soon as its own loads land): lane holds q~[16 nb + c][4E kb + E g + e]
        Frag qf[KBS][NB];
        if constexpr (!kFact) {
            const T *qb = reinterpret_cast<const T *>(p.q) + int64_t(b) * p.h * p.d_h;
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int head = 16 * nb + c;
                    const int d0 = 4 * E * kb + E * g;
                    qf[kb][nb] = M::load_q(qb, head, d0, p.h, p.d_h);
                }
        }
        // Two register stages (the next block's loads in flight while one is consumed) wherever they
        // fit in the register file; wide fp32 operands use one stage.
        constexpr bool kTwoStages = sizeof(T) == 2 || HP * DP <= 1024;
        Stage s0, s1;
        int blk = blk_begin + w;
        // The two stages are loaded unconditionally, clamped to the job's last block (which every wave
        // may read): a wave with a single block reads one block twice, but the loads then sit in fixed
        // program order, so the compiler can wait for each stage exactly instead of draining every load in
        // flight at the top of the pipelined loop below.
        // (Outside a fused step every work-group that gets here has a block.  A fused step's first job of an
        // empty sequence has none: its stages read the cache's first block instead and never use it, so that
        // no load sits behind a branch, which would leave every wait of the mode conservative.)
        const int last_blk = blk_end - 1;
        const bool any_blk = !kStep || blk_end > blk_begin;
        auto load_clamped = [&](Stage &st, int b) { load(st, b < last_blk ? b : last_blk, any_blk); };
        if (kTwoStages) {  // start streaming the first two blocks before anything else (a fused step issues
                           // the second after its own set-up: a wave cannot pass its loads' issue until most of
                           // them have landed, so work placed behind both stages would wait for the stream)
            load_clamped(s0, blk);
            if (kMode == kQRot) load_clamped(s1, blk + kWaves);
        }
        if constexpr (kFact) {
            // Factored query, while the first blocks stream in: q[i][d] = (1/R_Q) sum_r A_Q[r][i] B_Q[r][d]
            // (TPA notes page, tensor product decomposition applied to Q), computed once per work-group in
            // 4 x 4 register tiles from LDS, then rotated to the query's position len (RoPE is linear, so
            // rotating the combined row equals combining rotated B_Q rows: RoPE compatibility), all in fp32
            // (fp64 for fp32 queries), rounded once to the element type, and read back as this lane's
            // fragments.
            if (tid < DP / 2) rope_cos_sin<T>(sm_cs + 2 * tid, double(len), theta_j);
#pragma unroll
            for (int k = 0; k < QA_PER; ++k) {
                const int idx = tid + k * kThreads;
                if (idx < kMaxRQ * HP) sm_aq[idx / HP][idx % HP] = qa_raw[k];
            }
#pragma unroll
            for (int k = 0; k < QB_PER; ++k) {
                const int idx = tid + k * kThreads;
                if (idx < kMaxRQ * DP) sm_bq[idx / DP][idx % DP] = qb_raw[k];
            }
            __syncthreads();
            const float inv_rq = 1.f / float(p.r_q);
            for (int t = tid; t < (HP / 4) * (DP / 4); t += kThreads) {
                const int h0 = 4 * (t / (DP / 4)), d0 = 4 * (t % (DP / 4));
                float a4[4][4] = {};
                for (int r = 0; r < p.r_q; ++r) {
                    const float4 av = *reinterpret_cast<const float4 *>(&sm_aq[r][h0]);
                    const float4 bv = *reinterpret_cast<const float4 *>(&sm_bq[r][d0]);
                    const float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) a4[i][j] = fmaf(ar[i], br[j], a4[i][j]);
                }
                // features d0 .. d0 + 3 are the rotary pairs d0 / 2 and d0 / 2 + 1
                const F c0 = sm_cs[d0], s0 = sm_cs[d0 + 1], c1 = sm_cs[d0 + 2], s1 = sm_cs[d0 + 3];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    F y[4];
                    rope_rotate(F(a4[i][0]), F(a4[i][1]), c0, s0, y[0], y[1]);
                    rope_rotate(F(a4[i][2]), F(a4[i][3]), c1, s1, y[2], y[3]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float x = float(y[j] * F(inv_rq));
                        if constexpr (sizeof(T) == 2)
                            sm_q[h0 + i][d0 + j] = uint16_t(pack_bf16x2(x, 0.f) & 0xffffu);
                        else
                            sm_q[h0 + i][d0 + j] = x;
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) qf[kb][nb] = M::load(&sm_q[16 * nb + c][4 * E * kb + E * g]);
            if (kTwoStages) load_clamped(s1, blk + kWaves);
        }
        if constexpr (kStep) {
            // Fused step, while the first blocks stream in.  q arrives unrotated and sits at position len (the
            // number of cached tokens).  The first job stages the new token's factors in LDS and, after the one
            // barrier the angle table needs anyway, takes the token's score per head from the still unrotated
            // query fragments and the unrotated B_K: query and token share a position, so RoPE drops out of that
            // score (RoPE compatibility, Theorem 3.1 with t = s).  Then every wave rotates its query fragments
            // (the table covers every padded pair; theta is zero past d_h / 2: an identity rotation of zeros),
            // and the sequence's last job writes the token's record at slot len: no work-group of this kernel
            // reads that slot's rows (a partly filled last block masks every row at or past len), and the next
            // call sees it.
            // Over an E4M3 cache the token enters as its stored values, exactly as tpa_cache_append and then a
            // decode would see it: every factor is rounded to its code and decoded back, B_K after its rotation,
            // which no longer cancels in the score; so the first job stages the rotated, decoded B~_K after the
            // table and takes the score from the rotated query fragments behind a second barrier.
            auto token_score = [&]() {
                // the token's score per head: a lane sums its d-values, the four lane groups of a head are
                // summed across (the same contraction as the cached tokens'); head block nb is taken by wave
                // nb % kWaves, so the waves share the work
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (nb % kWaves != w) continue;  // wave-uniform; static register indexing
                    float dot[RH];
#pragma unroll
                    for (int r = 0; r < RH; ++r) {
                        float x = 0.f;
#pragma unroll
                        for (int kb = 0; kb < KBS; ++kb) {
                            float bk[E];
                            if constexpr (E == 8) {
                                const float4 lo = *reinterpret_cast<const float4 *>(&sm_nb[0][r][4 * E * kb + E * g]);
                                const float4 hi =
                                    *reinterpret_cast<const float4 *>(&sm_nb[0][r][4 * E * kb + E * g + 4]);
                                bk[0] = lo.x; bk[1] = lo.y; bk[2] = lo.z; bk[3] = lo.w;
                                bk[4] = hi.x; bk[5] = hi.y; bk[6] = hi.z; bk[7] = hi.w;
                            } else {
                                bk[0] = sm_nb[0][r][4 * E * kb + E * g];
                            }
#pragma unroll
                            for (int e = 0; e < E; ++e) x = fmaf(M::value(qf[kb][nb], e), bk[e], x);
                        }
                        dot[r] = wave_sum_across_groups(x);
                    }
                    if (g == 0) {
                        const int head = 16 * nb + c;
                        float z = 0.f;
#pragma unroll
                        for (int r = 0; r < RH; ++r) z = fmaf(sm_na[0][r][head], dot[r], z);
                        sm_m[kWaves][head] = head < p.h ? z * p.score_mul : -INFINITY;
                        sm_l[kWaves][head] = head < p.h ? 1.f : 0.f;
                    }
                }
            };
            // E4M3 codes of the token's items (A_K, A_V of this thread's head-factor item; B_V of its pair)
            uint32_t ak8 = 0, av8 = 0, bv8 = 0;
            if constexpr (kF8) {
                ak8 = e4m3_one(Elem<T>::to_f32(nak) * p.st.inv_scale[0]);
                av8 = e4m3_one(Elem<T>::to_f32(nav) * p.st.inv_scale[2]);
                bv8 = e4m3_pair(Elem<T>::to_f32(nbv0) * p.st.inv_scale[3], Elem<T>::to_f32(nbv1) * p.st.inv_scale[3]);
            }
            if (new_tok) {
                if (na_r < RH) {
                    if constexpr (kF8) {
                        sm_na[0][na_r][na_i] = __builtin_amdgcn_cvt_f32_fp8(int(ak8), 0);
                        sm_na[1][na_r][na_i] = __builtin_amdgcn_cvt_f32_fp8(int(av8), 0);
                    } else {
                        sm_na[0][na_r][na_i] = Elem<T>::to_f32(nak);
                        sm_na[1][na_r][na_i] = Elem<T>::to_f32(nav);
                    }
                }
                if (nb_r < RH) {
                    if constexpr (kF8) {
                        const floatx2 v = __builtin_amdgcn_cvt_pk_f32_fp8(int(bv8), false);
                        sm_nb[1][nb_r][nb_d] = v.x;
                        sm_nb[1][nb_r][nb_d + 1] = v.y;
                    } else {
                        sm_nb[0][nb_r][nb_d] = Elem<T>::to_f32(nbk0);
                        sm_nb[0][nb_r][nb_d + 1] = Elem<T>::to_f32(nbk1);
                        sm_nb[1][nb_r][nb_d] = Elem<T>::to_f32(nbv0);
                        sm_nb[1][nb_r][nb_d + 1] = Elem<T>::to_f32(nbv1);
                    }
                }
            }
            if (tid < DP / 2) rope_cos_sin<T>(sm_cs + 2 * tid, double(len), theta_j);
            __syncthreads();
            if constexpr (!kF8)
                if (new_tok) token_score();
#pragma unroll
            for (int kb = 0; kb < KBS; ++kb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) qf[kb][nb] = M::rotate_q(qf[kb][nb], 4 * E * kb + E * g, sm_cs);
            const int64_t slot = start + len;
            // the token's B~_K pair, rotated as tpa_cache_append rotates it
            F y0 = F(0), y1 = F(0);
            if ((kF8 ? (new_tok || rec_tok) : rec_tok) && nb_r < p.RK && nb_d < p.d_h)
                rope_rotate(F(Elem<T>::to_f32(nbk0)), F(Elem<T>::to_f32(nbk1)), sm_cs[nb_d], sm_cs[nb_d + 1], y0, y1);
            uint32_t bk8 = 0;
            if constexpr (kF8) {
                bk8 = e4m3_pair(float(y0) * p.st.inv_scale[1], float(y1) * p.st.inv_scale[1]);
                if (new_tok) {
                    if (nb_r < RH) {
                        const floatx2 v = __builtin_amdgcn_cvt_pk_f32_fp8(int(bk8), false);
                        sm_nb[0][nb_r][nb_d] = v.x;
                        sm_nb[0][nb_r][nb_d + 1] = v.y;
                    }
                    __syncthreads();  // first job only (uniform over the work-group)
                    token_score();
                }
            }
            if (rec_tok && slot < p.st.capacity) {
                const int row0 = int(slot % TOK) * RH;
                if constexpr (kF8) {
                    // the E4M3 record: the same codes tpa_cache_append writes, in the paired 8-bit layout
                    uint8_t *rec = reinterpret_cast<uint8_t *>(p.st.cache) + (slot / TOK) * BLK;
                    const Layout Lay = make_layout(p.h, p.d_h, p.RK, p.RV, Elem<T>::dtype, 1);
                    if (na_r < RH) {
                        rec[Lay.gate(row0 + na_r, na_i)] = uint8_t(ak8);
                        rec[OFF_AV + Lay.gate(row0 + na_r, na_i)] = uint8_t(av8);
                    }
                    if (nb_r < RH) {
                        *reinterpret_cast<uint16_t *>(rec + OFF_BK + Lay.bk(row0 + nb_r, nb_d)) = uint16_t(bk8);
                        rec[OFF_BV + Lay.bv(row0 + nb_r, nb_d)] = uint8_t(bv8 & 0xffu);
                        rec[OFF_BV + Lay.bv(row0 + nb_r, nb_d + 1)] = uint8_t(bv8 >> 8);
                    }
                } else {
                    // the record, B_K rotated and rounded exactly as tpa_cache_append stores it
                    T k0 = nbk0, k1 = nbk1;
                    if (nb_r < p.RK && nb_d < p.d_h) {
                        if constexpr (sizeof(T) == 2) {
                            const uint32_t pk = pack_bf16x2(y0, y1);
                            k0 = T(pk & 0xffffu);
                            k1 = T(pk >> 16);
                        } else {
                            k0 = T(y0);
                            k1 = T(y1);
                        }
                    }
                    T *rec = reinterpret_cast<T *>(p.st.cache) + (slot / TOK) * BLK;
                    const Layout Lay = make_layout(p.h, p.d_h, p.RK, p.RV, Elem<T>::dtype);
                    if (na_r < RH) {
                        rec[Lay.gate(row0 + na_r, na_i)] = nak;
                        rec[OFF_AV + Lay.gate(row0 + na_r, na_i)] = nav;
                    }
                    if (nb_r < RH) {
                        rec[OFF_BK + Lay.bk(row0 + nb_r, nb_d)] = k0;
                        rec[OFF_BK + Lay.bk(row0 + nb_r, nb_d + 1)] = k1;
                        rec[OFF_BV + Lay.bv(row0 + nb_r, nb_d)] = nbv0;
                        rec[OFF_BV + Lay.bv(row0 + nb_r, nb_d + 1)] = nbv1;
                    }
                }
            }
            if (kTwoStages) load_clamped(s1, blk + kWaves);
        }


        floatx4 acc[MBV][NB];
#pragma unroll
        for (int mv = 0; mv < MBV; ++mv)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mv][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
        // Scores are kept in raw units z = sum_r A_K U (the scale is applied inside the exponent);
        // run_m is the lazy reference max in raw units, neg_ms = -run_m * score_mul.
        float run_m[NB], neg_ms[NB], run_l[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            run_m[nb] = -INFINITY;
            neg_ms[nb] = INFINITY;
            run_l[nb] = 0.f;
        }
        const float sm = p.score_mul;
        const float lazy_raw = kLazy / sm;

        // Process one block.  kTail: the block may hold rows beyond the sequence (valid < TOK tokens);
        // only the last block of a sequence can, and it takes this slower masked path.
        auto process = [&](Stage &st, auto tail_tag, int valid) {
            constexpr bool kTail = decltype(tail_tag)::value;
            // ---- 1. score contraction
            floatx4 u[2][NB];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KBS; ++kb) a = M::mma(frag_bk(st, mb, kb), qf[kb][nb], a);
                    u[mb][nb] = a;
                }

            // ---- 2.-4. gates, online softmax, value weights
            float wv[2][NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float ak[2][4], av[2][4];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    gates(st, false, mb, nb, ak[mb]);
                    gates(st, true, mb, nb, av[mb]);
                }
                float z[2][TPL];
                float mx = -INFINITY;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int t = 0; t < TPL; ++t) {
                        float sc = ak[mb][t * RH] * u[mb][nb][t * RH];
#pragma unroll
                        for (int r = 1; r < RH; ++r) sc = fmaf(ak[mb][t * RH + r], u[mb][nb][t * RH + r], sc);
                        if (kTail) sc = (16 * mb + 4 * g) / RH + t < valid ? sc : -INFINITY;
                        z[mb][t] = sc;
                        mx = fmaxf(mx, sc);
                    }
                // Lazy reference max: the weights are taken relative to run_m, which only moves (with a
                // cross-lane max and a rescale of the accumulators) when some score exceeds it by more than
                // kLazy in log2 units, so p <= 2^kLazy and the common block needs no cross-lane traffic.
                if (__any(mx > run_m[nb] + lazy_raw)) {
                    const float mn = fmaxf(run_m[nb], wave_max_across_groups(mx));
                    const float alpha = __builtin_amdgcn_exp2f((run_m[nb] - mn) * sm);
                    run_m[nb] = mn;
                    neg_ms[nb] = -mn * sm;
                    run_l[nb] *= alpha;
#pragma unroll
                    for (int mv = 0; mv < MBV; ++mv) acc[mv][nb] *= alpha;
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int t = 0; t < TPL; ++t) {
                        const float pr = __builtin_amdgcn_exp2f(fmaf(z[mb][t], sm, neg_ms[nb]));
                        run_l[nb] += pr;
#pragma unroll
                        for (int r = 0; r < RH; ++r) {
                            float wgt = pr * av[mb][t * RH + r];
                            // rows beyond the sequence: p is 0 but the stored A_V may be anything
                            if (kTail) wgt = (16 * mb + 4 * g) / RH + t < valid ? wgt : 0.f;
                            wv[mb][nb][t * RH + r] = wgt;
                        }
                    }
            }

            // ---- 5. value contraction (in a tail block, rows beyond the sequence have arbitrary stored B_V:
            // their slots are zeroed in the operand)
#pragma unroll
            for (int q = 0; q < KBV; ++q) {
                unsigned bits = 0;
                if (kTail) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int t = E * q + e;
                        const int row = 16 * (t / 4) + 4 * g + (t % 4);
                        if (row / RH >= valid) bits |= 1u << e;
                    }
                }
                Frag bvf[MBV];
#pragma unroll
                for (int mv = 0; mv < MBV; ++mv)
                    bvf[mv] = kTail ? M::mask(frag_bv(st, mv, q), bits) : frag_bv(st, mv, q);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float x[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int t = E * q + e;
                        x[e] = wv[t / 4][nb][t % 4];
                    }
                    const Frag wf = M::pack(x);
#pragma unroll
                    for (int mv = 0; mv < MBV; ++mv) acc[mv][nb] = M::mma(bvf[mv], wf, acc[mv][nb]);
                    if constexpr (kSplitW) {  // the weights' bf16 rounding residuals, as a second product
                        float r[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) r[e] = x[e] - M::value(wf, e);
                        const Frag wl = M::pack(r);
#pragma unroll
                        for (int mv = 0; mv < MBV; ++mv) acc[mv][nb] = M::mma(bvf[mv], wl, acc[mv][nb]);
                    }
                }
            }
        };
        using Full = std::integral_constant<bool, false>;
        using Tail = std::integral_constant<bool, true>;

        // Steady state: stage k holds block blk + k * kWaves and both refills are real blocks, so the loop
        // issues the same loads in the same order every iteration and each stage waits for exactly its own
        // loads (with a conditional refill the compiler cannot count the loads issued after a stage and
        // drains everything in flight at the top of every iteration).
        if (kTwoStages) {
            while (blk + 3 * kWaves < full_end) {
                process(s0, Full{}, TOK);
                load(s0, blk + 2 * kWaves);
                process(s1, Full{}, TOK);
                load(s1, blk + 3 * kWaves);
                blk += 2 * kWaves;
            }
        }
        if (kTwoStages) {
            // The last (at most three) full blocks of the wave, in straight-line code so that the first one
            // still waits only for its own stage: blk in s0, blk + kWaves in s1, blk + 2 kWaves refilled
            // into s0.
            if (blk < full_end) {
                process(s0, Full{}, TOK);
                if (blk + 2 * kWaves < full_end) load(s0, blk + 2 * kWaves);
                blk += kWaves;
                if (blk < full_end) {
                    process(s1, Full{}, TOK);
                    blk += kWaves;
                    if (blk < full_end) {
                        process(s0, Full{}, TOK);
                        blk += kWaves;
                    }
                }
            }
        } else {
            for (; blk < full_end; blk += kWaves) {
                load(s0, blk);
                process(s0, Full{}, TOK);
            }
        }
        // the sequence's last, partly filled block, if it falls to this wave
        if (blk < blk_end) {
            load(s0, blk);
            process(s0, Tail{}, len - blk * TOK);
        }
        // back to log2 units for the merges
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) run_m[nb] = run_m[nb] * sm;

        // ---- merge the waves of this work-group
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) run_l[nb] = wave_sum_across_groups(run_l[nb]);
        if (g == 0) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                sm_m[w][16 * nb + c] = run_m[nb];
                sm_l[w][16 * nb + c] = run_l[nb];
            }
        }
        __syncthreads();
        float wscale[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int head = 16 * nb + c;
            float mm = sm_m[0][head];
#pragma unroll
            for (int ww = 1; ww <= kWaves; ++ww) mm = fmaxf(mm, sm_m[ww][head]);
            wscale[nb] = run_m[nb] == -INFINITY ? 0.f : exp2f(run_m[nb] - mm);
            if constexpr (kStep)
                if (new_tok && w == 0 && g == 0)  // the new token's weight, once per head
                    sm_wt[head] = sm_m[kWaves][head] == -INFINITY ? 0.f : exp2f(sm_m[kWaves][head] - mm);
        }
        // every wave writes its rescaled accumulators to its own LDS slice; after one barrier all threads
        // sum the slices column by column straight into the job's partial
#pragma unroll
        for (int mv = 0; mv < MBV; ++mv)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const floatx4 a = acc[mv][nb] * wscale[nb];
                *reinterpret_cast<float4 *>(&sm_o[w][16 * nb + c][16 * mv + 4 * g]) =
                    make_float4(a[0], a[1], a[2], a[3]);
            }
        __syncthreads();
        // write the job's partial: O [HP][DP], (max, sum) [HP]
        float *wo = p.ws_o + part * HP * DP;
        for (int idx = threadIdx.x; idx < HP * DP / 4; idx += kThreads) {
            const int hh = idx / (DP / 4), d4 = idx % (DP / 4);
            float4 o = *reinterpret_cast<const float4 *>(&sm_o[0][hh][4 * d4]);
#pragma unroll
            for (int ww = 1; ww < kWaves; ++ww) {
                const float4 x = *reinterpret_cast<const float4 *>(&sm_o[ww][hh][4 * d4]);
                o.x += x.x;
                o.y += x.y;
                o.z += x.z;
                o.w += x.w;
            }
            if constexpr (kStep) {
                if (new_tok) {  // the new token's value row, at its own weight
                    const float wt = sm_wt[hh];
                    float v[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int r = 0; r < RH; ++r)
#pragma unroll
                        for (int k = 0; k < 4; ++k) v[k] = fmaf(sm_na[1][r][hh], sm_nb[1][r][4 * d4 + k], v[k]);
                    o.x = fmaf(v[0], wt, o.x);
                    o.y = fmaf(v[1], wt, o.y);
                    o.z = fmaf(v[2], wt, o.z);
                    o.w = fmaf(v[3], wt, o.w);
                }
            }
            *reinterpret_cast<float4 *>(wo + hh * DP + 4 * d4) = o;
        }
        for (int head = threadIdx.x; head < HP; head += kThreads) {
            float mm = sm_m[0][head];
            for (int ww = 1; ww <= kWaves; ++ww) mm = fmaxf(mm, sm_m[ww][head]);
            float ll = 0.f;
            for (int ww = 0; ww <= kWaves; ++ww)
                ll += sm_m[ww][head] == -INFINITY ? 0.f : sm_l[ww][head] * exp2f(sm_m[ww][head] - mm);
            *reinterpret_cast<float2 *>(p.ws_ml + (part * HP + head) * 2) = make_float2(mm, ll);
        }
    };

    // the jobs of this work-group's range, in batch order
    int b = __builtin_amdgcn_readfirstlane(sm_first[0]);
    int Vb = __builtin_amdgcn_readfirstlane(sm_first[1]);
    for (bool first_of_wg = true;; first_of_wg = false) {
        SeqInfo si;
        if (first_of_wg) {
            si.len = sm_first_len;
            si.vb = sm_first_vb;
            si.start = sm_first_start;
            si.rejected = sm_first_rej != 0;
        } else {
            si = seq_info(b);
        }
        const int vb = stride > 0 ? stride : si.vb;  // the sequence's share of the partition
        const int lo = max(gs, Vb) - Vb, hi = min(ge, Vb + vb) - Vb;
        const bool first_job = Vb >= gs, last_job = Vb + vb <= ge;
        // the work-group of a sequence's first block records the range of work-groups that hold its pieces
        if (first_job && tid == 0) p.ws_meta[b] = make_int2(wg, int((Vb + vb - 1) / per_wg));
        run_job(b, si, int64_t(wg) + b, lo, hi, first_job, last_job);
        Vb += vb;
        if (Vb >= ge || ++b >= p.batch) break;
        __syncthreads();  // the next job reuses this one's LDS
    }
}

// Second pass: merge the partials of each sequence's pieces.  One work-group of kThr threads per (head,
// sequence); thread t owns output columns 4 (t % C4) .. +3 and the pieces j = t / C4 (mod JL),
// where C4 = DP / 4 and JL = kThr / C4.  Each thread folds its pieces with the
// same rescaling rule, loads issued eight at a time, and the JL lanes of a column
// group are folded once more through LDS.  (A fused step's new token is already part
// of the first piece's partial.)  The launch takes 128 threads when the planner expects every lane to
// have one round of loads (a short call: the smaller work-group finishes sooner), else 256.
constexpr int kMergeUnroll = 8;

template <int kThr>
__global__ __launch_bounds__(kThr) void decode_merge_kernel(DecodeParams p, int HP, int DP, int TOK) {
    __shared__ float sm[kThr][6];
    const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int C4 = DP / 4, JL = kThr / C4;
    const int c4 = tid % C4, jl = tid / C4;
    // The sequence's pieces sit at partial indices wg + b for the work-groups wg its meta record names
    // (every one of them wrote a partial; an empty one has max -inf).  Start and length only decide the
    // rejected case (the split kernel's predicate).
    const int2 wgs = p.ws_meta[b];
    const int64_t start = p.seq_start[b];
    int len = p.seq_len[b];
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    const bool rejected = seq_rejected(start, int64_t(len) + (p.step ? 1 : 0), TOK, p.capacity);
    const int n_valid = wgs.y - wgs.x + 1;

    float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    const int64_t base = int64_t(wgs.x) + b;
    for (int j0 = jl; j0 < n_valid; j0 += JL * kMergeUnroll) {
        float mj[kMergeUnroll], lj[kMergeUnroll];
        float4 oj[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int j = j0 + u * JL;
            if (j < n_valid) {
                const int64_t part = base + j;
                const float2 ml = *reinterpret_cast<const float2 *>(p.ws_ml + (part * HP + head) * 2);
                mj[u] = ml.x;
                lj[u] = ml.y;
                oj[u] = *reinterpret_cast<const float4 *>(p.ws_o + (part * HP + head) * DP + 4 * c4);
            } else {
                mj[u] = -INFINITY;
                lj[u] = 0.f;
                oj[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            if (mj[u] == -INFINITY) continue;
            const float Mn = fmaxf(M, mj[u]);
            const float a = exp2f(M - Mn), c = exp2f(mj[u] - Mn);
            L = L * a + lj[u] * c;
            o0 = o0 * a + oj[u].x * c;
            o1 = o1 * a + oj[u].y * c;
            o2 = o2 * a + oj[u].z * c;
            o3 = o3 * a + oj[u].w * c;
            M = Mn;
        }
    }
    sm[tid][0] = M;
    sm[tid][1] = L;
    sm[tid][2] = o0;
    sm[tid][3] = o1;
    sm[tid][4] = o2;
    sm[tid][5] = o3;
    __syncthreads();
    if (jl != 0 || head >= p.h || 4 * c4 >= p.d_h) return;
    for (int k = 1; k < JL; ++k) {
        const float *r = sm[tid + k * C4];
        if (r[0] == -INFINITY) continue;
        const float Mn = fmaxf(M, r[0]);
        const float a = exp2f(M - Mn), c = exp2f(r[0] - Mn);
        L = L * a + r[1] * c;
        o0 = o0 * a + r[2] * c;
        o1 = o1 * a + r[3] * c;
        o2 = o2 * a + r[4] * c;
        o3 = o3 * a + r[5] * c;
        M = Mn;
    }
    float o[4] = {o0, o1, o2, o3};
    if (rejected) {
        o[0] = o[1] = o[2] = o[3] = __builtin_nanf("");
    } else if (L == 0.f) {  // no tokens
        o[0] = o[1] = o[2] = o[3] = 0.f;
    } else {
        const float inv = p.out_mul / L;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] *= inv;
    }
    float *out = p.out + (int64_t(b) * p.h + head) * p.d_h;
    for (int k = 0; k < 4 && 4 * c4 + k < p.d_h; ++k) out[4 * c4 + k] = o[k];
}

template <typename T, int HP, int DP, int RH>
hipError_t launch_split(const DecodeParams &p, bool f8, hipStream_t s) {
    const dim3 grid(p.grid);
    if constexpr (sizeof(T) == 2) {
        if (f8) {
            if (p.step)
                hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kStepMode, true>), grid, dim3(kThreads), 0, s, p);
            else if (p.r_q > 0)
                hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kQFact, true>), grid, dim3(kThreads), 0, s, p);
            else
                hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kQRot, true>), grid, dim3(kThreads), 0, s, p);
            return hipGetLastError();
        }
    }
    if (f8) return hipErrorInvalidValue;
    if (p.step)
        hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kStepMode, false>), grid, dim3(kThreads), 0, s, p);
    else if (p.r_q > 0)
        hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kQFact, false>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<T, HP, DP, RH, kQRot, false>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T, int HP, int DP>
hipError_t launch_split_rank(int RH, const DecodeParams &p, bool f8, hipStream_t s) {
    switch (RH) {
        case 1: return launch_split<T, HP, DP, 1>(p, f8, s);
        case 2: return launch_split<T, HP, DP, 2>(p, f8, s);
        case 4: return launch_split<T, HP, DP, 4>(p, f8, s);
    }
    return hipErrorInvalidValue;
}

// Compiled (element type, padded heads, padded head dim) combinations.
#define TPA_DECODE_SHAPES(X)                                                                            \
    X(uint16_t, 2, 16, 32) X(uint16_t, 2, 16, 64) X(uint16_t, 2, 16, 128) X(uint16_t, 2, 32, 32)     \
        X(uint16_t, 2, 32, 64) X(uint16_t, 2, 32, 128) X(uint16_t, 2, 64, 32) X(uint16_t, 2, 64, 64) \
            X(float, 4, 16, 16) X(float, 4, 16, 32) X(float, 4, 16, 64) X(float, 4, 16, 128)         \
                X(float, 4, 32, 32) X(float, 4, 32, 64) X(float, 4, 32, 128)

}  // namespace

int decode_merge_threads(const Layout &L, const DecodeParams &p) {
    return p.merge_parts <= (128 / (L.DP / 4)) * kMergeUnroll ? 128 : 256;
}

// An E4M3 cache runs the bf16 shapes (its operands are bf16 after decoding).
bool decode_supported(const Layout &L) {
    const int es = L.f8 ? 2 : L.es;
#define X(T, ES, HP_, DP_) \
    if (es == ES && L.HP == HP_ && L.DP == DP_) return true;
    TPA_DECODE_SHAPES(X)
#undef X
    return false;
}

hipError_t launch_decode(const Layout &L, const DecodeParams &p, hipStream_t s) {
    hipError_t e = hipErrorInvalidValue;
    bool found = false;
    const int es = L.f8 ? 2 : L.es;
#define X(T, ES, HP_, DP_)                                         \
    if (!found && es == ES && L.HP == HP_ && L.DP == DP_) {         \
        found = true;                                              \
        e = launch_split_rank<T, HP_, DP_>(L.RH, p, L.f8 != 0, s); \
    }
    TPA_DECODE_SHAPES(X)
#undef X
    if (!found || e != hipSuccess) return e;
    if (decode_merge_threads(L, p) == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(L.HP, p.batch), dim3(128), 0, s, p, L.HP, L.DP,
                           L.tok_per_block());
    else
        hipLaunchKernelGGL(decode_merge_kernel<256>, dim3(L.HP, p.batch), dim3(256), 0, s, p, L.HP, L.DP,
                           L.tok_per_block());
    return hipGetLastError();
}

}  // namespace tpa
