// Causal chunked prefill over a TPA factor cache.
//
// TPA notes page, Key design: K_s = (1/R_K) A_K[s]^T B_K[s] and V_s likewise;
// FlashTPA: no full K/V in device memory.  A prefill chunk has many query
// rows per head, so each work-group rebuilds one head's key and value rows of
// a 64-token tile on chip,
//     K~_i[s,:] = sum_r A_K[s,r,i] B~_K[s,r,:]      (1/R_K folded into the scale)
//     V_i[s,:]  = sum_r A_V[s,r,i] B_V[s,r,:]       (1/R_V applied at the end)
// in fp32 from the cached factors, rounds them once to bf16 into LDS, and
// runs a flash-attention loop on the bf16 matrix cores (32x32x16).  At rank 1
// the rows in LDS are the cached B~_K and B_V themselves (no rounding), and the
// gates A_K[s,0,i] and A_V[s,0,i] multiply the scores and the softmax weights in
// fp32; the weights p A_V reach the matrix cores as a bf16 pair hi + lo (two
// products with the same V^T operand), and the row sum takes the fp32 p, so
// the kernel adds nothing to the rounding of the values it reads.
//     S^T = K~_i Q~^T   (M = keys, N = queries, K = d_h)
//     causal mask: chunk row j (position ctx + j) sees keys 0 .. ctx + j
//     online softmax per query (a lane owns one query column)
//     O^T += V_i^T P^T  (M = d_h, N = queries, K = keys)
// A work-group owns 256 query rows of one head (8 waves x 32), so every
// (key, head) pair is rebuilt at most twice per chunk of 512 rows; chunks of
// more than 256 rows at d_h = 128 and rank 2 or 4 take the wide form further down (512 rows
// per work-group, factor pieces staged in LDS by direct loads).  The LDS
// tiles are double-buffered: the factor loads of a later tile are issued between
// the matrix-core instructions of tile t, and the waves rebuild tile t+1 (half of
// them at the end of their iteration, half at its start: see prefill_kernel).  The key order inside the value contraction is
// permuted (bits 2 and 3 of the key index swapped within each group of 16)
// so that the score accumulator a lane holds is exactly its slice of P^T and
// its slice of V^T is one 16-byte LDS read.
#include <type_traits>

#include "common.h"

namespace tpa {
namespace {

constexpr int kPrefillWaves = 8;
static_assert(kPrefillThreads == kPrefillWaves * kWave, "one prefill work-group is 8 waves");
constexpr int kQT = 32 * kPrefillWaves;  // query rows per work-group
static_assert(kQT == kPrefillRows, "the launch planner sizes grids by these rows");
constexpr int kKT = 64;                  // keys per tile
constexpr float kLazyPrefill = 8.0f;     // headroom of the lazy reference max, log2 units
constexpr int kXcds = 8;                 // MI355X: 8 XCDs, 32 CUs and one L2 each

__device__ __forceinline__ floatx16 mma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    const uint4 v = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// LDS position of tile key k inside the value contraction's key order
__device__ __forceinline__ int vpos(int k) { return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3); }

// Factored query row (tpa_prefill_chunk_fq): the MFMA B-operand fragments of query row jq that a lane of
// a 32x32x16 product supplies (features 16 ks + 8 hi + e, e < 8):
//     q[d] = (1/R_Q) sum_r A_Q[jq][r][head] B_Q[jq][r][d]    (TPA notes page, tensor product decomposition
//                                                             applied to Q)
// summed in fp32, then rotated to the row's position pos (RoPE is linear, so rotating the combined row equals
// combining rotated B_Q rows), and rounded once to bf16.  Rows past the chunk are zeros.  The angle
// pos * theta_j is reduced in fp64 to a fraction of a turn, whose sine and cosine come from the hardware
// v_sin_f32 / v_cos_f32 (absolute error ~1e-6, far below the bf16 rounding that follows); the library's
// sincosf would be as exact as the append's, but 32 of them per row block overflow the register budget of
// the wide form into scratch memory.
template <int KS>
__device__ __forceinline__ void factored_query_row(const PrefillParams &p, int b, int jq, int head, int hi, int pos,
                                                   bf16x8 *qf) {
    constexpr double kInvTwoPi = 0.15915494309189535;
    constexpr int KH = KS / 2;  // fragments per half
    const bool row = jq < p.chunk;
    const int64_t rw = int64_t(b) * p.chunk + jq;
    const uint16_t *aq = reinterpret_cast<const uint16_t *>(p.a_q) + rw * p.r_q * p.h + head;
    const uint16_t *bq = reinterpret_cast<const uint16_t *>(p.q) + rw * p.r_q * p.d_h;
    const float inv_rq = 1.f / float(p.r_q);
    const bool vec = (p.d_h & 7) == 0;
    // Half the fragments at a time (their 8 KH sums live), two factor rows per round of loads: every load of a
    // round is issued before any is used, so the build costs R_Q rounds of load latency in all.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float x[KH][8];
#pragma unroll
        for (int k = 0; k < KH; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[k][e] = 0.f;
        if (row) {
            for (int r = 0; r < p.r_q; r += 2) {
                const bool two = r + 1 < p.r_q;
                const float a0 = bf16_to_f32(aq[r * p.h]);
                const float a1 = two ? bf16_to_f32(aq[(r + 1) * p.h]) : 0.f;
                uint4 v0[KH], v1[KH];
#pragma unroll
                for (int k = 0; k < KH; ++k) {
                    const int d0 = 16 * (half * KH + k) + 8 * hi;
                    v0[k] = v1[k] = make_uint4(0, 0, 0, 0);
                    if (vec && d0 < p.d_h) {
                        v0[k] = *reinterpret_cast<const uint4 *>(bq + r * p.d_h + d0);
                        if (two) v1[k] = *reinterpret_cast<const uint4 *>(bq + (r + 1) * p.d_h + d0);
                    }
                }
#pragma unroll
                for (int k = 0; k < KH; ++k) {
                    const int d0 = 16 * (half * KH + k) + 8 * hi;
                    const uint32_t w0[4] = {v0[k].x, v0[k].y, v0[k].z, v0[k].w};
                    const uint32_t w1[4] = {v1[k].x, v1[k].y, v1[k].z, v1[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float b0, b1;
                        if (vec) {
                            b0 = __uint_as_float((e & 1) ? (w0[e >> 1] & 0xffff0000u) : (w0[e >> 1] << 16));
                            b1 = __uint_as_float((e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16));
                        } else {  // head dims that are not a multiple of 8: element by element
                            b0 = d0 + e < p.d_h ? bf16_to_f32(bq[r * p.d_h + d0 + e]) : 0.f;
                            b1 = two && d0 + e < p.d_h ? bf16_to_f32(bq[(r + 1) * p.d_h + d0 + e]) : 0.f;
                        }
                        x[k][e] = fmaf(a1, b1, fmaf(a0, b0, x[k][e]));
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KH; ++k)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int d = 16 * (half * KH + k) + 8 * hi + e;  // even: the pair (d, d + 1)
                    if (d < p.d_h) {
                        const double turns = double(pos) * (p.rope.theta[d >> 1] * kInvTwoPi);
                        const float t = float(turns - rint(turns));  // in [-1/2, 1/2]
                        const float c = __builtin_amdgcn_cosf(t), sn = __builtin_amdgcn_sinf(t);
                        float y0, y1;
                        rope_rotate(x[k][e], x[k][e + 1], c, sn, y0, y1);
                        x[k][e] = y0 * inv_rq;
                        x[k][e + 1] = y1 * inv_rq;
                    }
                }
        }
#pragma unroll
        for (int k = 0; k < KH; ++k) qf[half * KH + k] = pack8(x[k]);
    }
}

// kFQ: the query rows arrive as factors (tpa_prefill_chunk_fq), a separate instantiation.
// The double-buffered K~ and V^T tiles (row strides padded by 8 elements against bank conflicts).
// kGate (rank 1): the tiles hold the cached B~_K and B_V rows as they are, and each key's A_K and A_V gates
// (fp32) sit beside them, applied to the scores and to the softmax weights in fp32.  (A K~ row rebuilt as
// A_K B~_K and rounded to bf16 would move a sharp softmax by 2^-9 of its largest value rows.)
template <int DP, bool kGate>
struct PrefillLds {
    uint16_t k[2][kKT * (DP + 8)];
    uint16_t v[2][DP * (kKT + 8)];
    float gk[2][kGate ? kKT : 0];  // zero-length when unused (a clang extension)
    float gv[2][kGate ? kKT : 0];
};

// One work-group's loop.  late: the second wave of each SIMD (waves 4..7), which rebuilds at the top of
// its iteration instead of the end; see prefill_kernel.
template <int HP, int DP, int RH, bool kFQ, bool late, bool kF8>
__device__ __forceinline__ void prefill_body(const PrefillParams &p, PrefillLds<DP, RH == 1> &lds) {
    auto &sK = lds.k;
    auto &sV = lds.v;
    constexpr int KS = DP / 16;  // score K steps
    constexpr int MB = DP / 32;  // value M blocks
    constexpr int NB = HP / 16;
    constexpr int KBS = DP / 32;  // B~_K 32-wide column blocks in the cache layout
    constexpr int MBV = DP / 16;
    constexpr int TOK = kRows / RH;
    constexpr bool kGate = RH == 1;  // gates applied in fp32 (see PrefillLds)
    constexpr int SKS = DP + 8;   // LDS row stride of K~ (bf16 elements)
    constexpr int SVS = kKT + 8;  // LDS row stride of V^T
    constexpr int BLK = 2 * kRows * (HP + DP);
    constexpr int OFF_AV = kRows * HP, OFF_BK = 2 * kRows * HP, OFF_BV = 2 * kRows * HP + kRows * DP;

    // Work-groups are dispatched round-robin over the 8 XCDs (linear id mod 8), each with its own L2.
    // When the batch is a multiple of 8, the linear id is mapped so that all work-groups of a sequence
    // (every head and query tile: they all read the same B factors) land on one XCD and share its L2.
    const int n_qt = (p.chunk + kQT - 1) / kQT;
    const int L = blockIdx.x;
    int b, head, qt;
    if (p.batch % kXcds == 0) {
        const int per_seq = p.h * n_qt;
        b = L % kXcds + kXcds * (L / (kXcds * per_seq));
        const int r = (L / kXcds) % per_seq;
        head = r / n_qt;
        qt = r % n_qt;
    } else {
        qt = L % n_qt;
        head = (L / n_qt) % p.h;
        b = L / (n_qt * p.h);
    }
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hi = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j0 = qt * kQT;
    const int jw = j0 + 32 * w;  // first query row of this wave
    const int jq = jw + col;     // query row of this lane's accumulator column
    int ctx = p.ctx_len[b];
    const int64_t start = p.seq_start[b];
    ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
    float *out = p.out + int64_t(b) * p.chunk * p.h * p.d_h;

    // a misaligned sequence, or one whose context and chunk reach past the capacity: NaN, nothing read
    if (seq_rejected(start, int64_t(ctx) + p.chunk, TOK, p.capacity)) {
        for (int idx = tid; idx < kQT * p.d_h; idx += kPrefillThreads) {
            const int j = j0 + idx / p.d_h, d = idx % p.d_h;
            if (j < p.chunk) out[(int64_t(j) * p.h + head) * p.d_h + d] = __builtin_nanf("");
        }
        return;
    }
    constexpr uint32_t CES = kF8 ? 1u : 2u;  // bytes per stored element (E4M3 codes, or bf16)
    const char *seq = reinterpret_cast<const char *>(p.cache) + (start / TOK) * int64_t(BLK) * CES;
    const int j_last = min(p.chunk, j0 + kQT) - 1;
    const int n_keys = ctx + j_last + 1;  // keys any row of this work-group sees (all appended)
    const int n_kt = (n_keys + kKT - 1) / kKT;
    const int gate_lane = head & 15, gate_nb = head >> 4;

    // ---- rebuild of K~_i and V_i^T for one tile.  Each thread owns fixed items; since a tile starts
    // at a block boundary, every load address is the tile's first block plus a per-thread constant
    // (computed once here) plus a compile-time step per item.  All loads of a tile are issued before
    // any arithmetic; products are bf16 pairs fed to v_dot2_f32_bf16 (fp32 accumulation).
    constexpr int C8 = DP / 8;                                    // 8-feature chunks per key row
    constexpr int K_ITEMS = kKT * C8 / kPrefillThreads;           // (key, 8 features) per thread
    constexpr int K_STEP = kPrefillThreads / C8;                  // keys between a thread's items
    // V items: the 8 wave-rows of the group split over the tile's blocks; a thread takes one block and
    // one chunk lane, and V_ITEMS feature groups of that block, so it needs one pair of gate loads
    constexpr int BPT = kKT / TOK;                                // cache blocks per tile
    constexpr int MVG = kPrefillWaves / BPT;                      // thread rows sharing one block
    constexpr int V_ITEMS = MBV / MVG;                            // 16-feature groups per thread
    static_assert(K_ITEMS * kPrefillThreads == kKT * C8 && K_STEP % TOK == 0, "K items must tile the group");
    static_assert(MVG * BPT == kPrefillWaves && V_ITEMS * MVG == MBV, "V items must tile the group");
    const int kk = tid / C8, c8 = tid % C8;    // key of item 0, its feature chunk
    const int krow0 = (kk % TOK) * RH;         // the key's first factor row in its block
    const int kv0 = krow0 & 3;                 // its first gate inside a 4-gate chunk
    // byte offsets from the tile's first block (unsigned 32-bit: scalar base + vector offset addressing).
    // An E4M3 cache stores the same pieces at one byte per element, paired per lane (gates: both row
    // blocks; B~_K: both row blocks of a k-block; B_V: value blocks 2j, 2j+1).
    const uint32_t k_off_blk = uint32_t((kk / TOK) * BLK) * CES;  // block of item 0 inside the tile
    const int k_mb = krow0 >> 4, k_gl = 16 * ((krow0 & 15) >> 2) + gate_lane;
    const uint32_t k_off_gate =
        k_off_blk + (kF8 ? uint32_t(((gate_nb * kWave + k_gl) * 2 + k_mb) * 4)
                         : uint32_t(((k_mb * NB + gate_nb) * kWave + k_gl) * 4) * 2u);
    uint32_t k_off_b[RH];
#pragma unroll
    for (int r = 0; r < RH; ++r) {
        const int row = krow0 + r, d0 = 8 * c8;
        const int kb = d0 >> 5, bl = 16 * ((d0 & 31) >> 3) + (row & 15);
        k_off_b[r] = k_off_blk + (kF8 ? uint32_t(OFF_BK + ((kb * kWave + bl) * 2 + (row >> 4)) * 8)
                                      : uint32_t(OFF_BK + (((row >> 4) * KBS + kb) * kWave + bl) * 8) * 2u);
    }
    const int vrow = tid / kWave, vcl = tid % kWave, vg4 = vcl >> 4;
    const int vbi = vrow % BPT, vmv0 = (vrow / BPT) * V_ITEMS;  // block inside the tile, first feature group
    // E4M3: with an even item count (vmv0 even) a thread loads its value chunks two at a time (one
    // 16-byte pair piece); a single item loads its own 8 bytes of the pair piece.
    constexpr bool VPAIR = V_ITEMS % 2 == 0;
    // feature of item u: 16 (vmv0 + u) + vcl % 16; chunk of item u: (vmv0 + u) * 64 + vcl
    const uint32_t v_off = kF8 ? uint32_t(vbi * BLK + OFF_BV + (((vmv0 >> 1) * kWave + vcl) * 2 + (VPAIR ? 0 : (vmv0 & 1))) * 8)
                               : uint32_t(vbi * BLK + OFF_BV + (vmv0 * kWave + vcl) * 8) * 2u;
    const int v_gl = 16 * vg4 + gate_lane;
    const uint32_t v_off_gate = kF8 ? uint32_t(vbi * BLK + OFF_AV + (gate_nb * kWave + v_gl) * 8)
                                    : uint32_t(vbi * BLK + OFF_AV + (gate_nb * kWave + v_gl) * 4) * 2u;

    // raw factor data of one tile, in registers between its loads and its rebuild
    struct RawNative {
        uint2 kg[K_ITEMS];
        uint4 kb_raw[K_ITEMS][RH];
        uint4 vx[V_ITEMS];
        uint2 vg[2];
    };
    struct RawF8 {  // E4M3 codes: 4 gates per word, 8 features per uint2, two value chunks per uint4
        uint32_t kg[K_ITEMS];
        uint2 kb_raw[K_ITEMS][RH];
        uint4 vx[VPAIR ? V_ITEMS / 2 : 1];
        uint2 vx1;  // single-item case
        uint2 vg;
    };
    using Raw = std::conditional_t<kF8, RawF8, RawNative>;
    // the rebuild's inputs as bf16 (E4M3 codes decode exactly to bf16)
    auto in_kg = [&](const Raw &raw, int u) -> uint2 {
        if constexpr (kF8) return e4m3x4_to_bf16x4(raw.kg[u]);
        else return raw.kg[u];
    };
    auto in_kb = [&](const Raw &raw, int u, int r) -> uint4 {
        if constexpr (kF8) return e4m3x8_to_bf16x8(raw.kb_raw[u][r].x, raw.kb_raw[u][r].y);
        else return raw.kb_raw[u][r];
    };
    auto in_vx = [&](const Raw &raw, int u) -> uint4 {
        if constexpr (kF8) {
            if constexpr (!VPAIR) return e4m3x8_to_bf16x8(raw.vx1.x, raw.vx1.y);
            const uint4 w = raw.vx[u >> 1];
            return (u & 1) ? e4m3x8_to_bf16x8(w.z, w.w) : e4m3x8_to_bf16x8(w.x, w.y);
        } else {
            return raw.vx[u];
        }
    };
    auto in_vg = [&](const Raw &raw, int m) -> uint2 {
        if constexpr (kF8) return e4m3x4_to_bf16x4(m ? raw.vg.y : raw.vg.x);
        else return raw.vg[m];
    };
    // Loads of one tile, in two halves (the K~ inputs, the V inputs) so that each half can be issued
    // between the matrix-core instructions of one phase.  Only the last tile may reach past n_keys:
    // there a block past the last live one is replaced by that block (its keys are zeroed in the
    // rebuild), so no address leaves the sequence's slots.  No branches: the selects keep each half in
    // the basic block it is placed in.
    auto tile_base = [&](int kt) { return seq + int64_t((kt * kKT) / TOK) * BLK * CES; };  // tile's first block
    auto tile_last_blk = [&](int kt) {  // last block with live keys, tile-relative (large if the tile is whole)
        const int key0 = kt * kKT;
        return key0 + kKT <= n_keys ? 1 << 20 : (n_keys - 1) / TOK - key0 / TOK;
    };
    auto fetch_k = [&](Raw &raw, int kt) {
        const char *tb = tile_base(kt);
        const int last_blk = tile_last_blk(kt);
#pragma unroll
        for (int u = 0; u < K_ITEMS; ++u) {
            // item u's block lies u * (K_STEP / TOK) blocks past item 0's
            const uint32_t delta = uint32_t(min(kk / TOK + u * (K_STEP / TOK), last_blk) * BLK) * CES - k_off_blk;
            if constexpr (kF8) {
                raw.kg[u] = *reinterpret_cast<const uint32_t *>(tb + (k_off_gate + delta));
#pragma unroll
                for (int r = 0; r < RH; ++r) raw.kb_raw[u][r] = *reinterpret_cast<const uint2 *>(tb + (k_off_b[r] + delta));
            } else {
                raw.kg[u] = *reinterpret_cast<const uint2 *>(tb + (k_off_gate + delta));
#pragma unroll
                for (int r = 0; r < RH; ++r) raw.kb_raw[u][r] = *reinterpret_cast<const uint4 *>(tb + (k_off_b[r] + delta));
            }
        }
    };
    auto fetch_v = [&](Raw &raw, int kt) {
        const char *tb = tile_base(kt);
        const uint32_t delta = uint32_t((min(vbi, tile_last_blk(kt)) - vbi) * BLK) * CES;
        if constexpr (kF8) {
            if constexpr (VPAIR) {
#pragma unroll
                for (int u2 = 0; u2 < V_ITEMS / 2; ++u2)
                    raw.vx[u2] = *reinterpret_cast<const uint4 *>(tb + (v_off + uint32_t(u2 * kWave * 16) + delta));
            } else {
                static_assert(V_ITEMS == 1, "odd item counts are single items");
                raw.vx1 = *reinterpret_cast<const uint2 *>(tb + (v_off + delta));
            }
            raw.vg = *reinterpret_cast<const uint2 *>(tb + (v_off_gate + delta));
        } else {
#pragma unroll
            for (int u = 0; u < V_ITEMS; ++u)
                raw.vx[u] = *reinterpret_cast<const uint4 *>(tb + (v_off + uint32_t(u * kWave * 8 * 2) + delta));
#pragma unroll
            for (int m = 0; m < 2; ++m)
                raw.vg[m] = *reinterpret_cast<const uint2 *>(tb + (v_off_gate + uint32_t(m * NB * kWave * 4 * 2) + delta));
        }
    };
    // Partial: true only for a tile that reaches past n_keys (its dead keys are written as zeros).
    auto rebuild = [&](Raw &raw, int kt, int buf, auto partial_tag) {
        constexpr bool kPartial = decltype(partial_tag)::value;
        const int key0 = kt * kKT;
        uint16_t *dK = sK[buf];
        uint16_t *dV = sV[buf];
        // -- K~ rows: K~[key][d] = sum_r A_K[key][r] B~_K[key][r][d]
#pragma unroll
        for (int u = 0; u < K_ITEMS; ++u) {
            const int k = kk + u * K_STEP;
            const uint2 kgu = in_kg(raw, u);
            const uint32_t gw[2] = {kgu.x, kgu.y};
            if constexpr (kGate) {
                // the cached row itself; the key's gate beside it (written by the thread of its first chunk)
                const bool dead = kPartial && key0 + k >= n_keys;
                const uint4 row = in_kb(raw, u, 0);
                const uint32_t a = (kv0 & 1) ? (gw[kv0 >> 1] >> 16) : (gw[kv0 >> 1] & 0xffffu);
                if (c8 == 0) lds.gk[buf][k] = dead ? 0.f : __builtin_bit_cast(float, a << 16);
                *reinterpret_cast<uint4 *>(&dK[k * SKS + 8 * c8]) = dead ? make_uint4(0, 0, 0, 0) : row;
                continue;
            }
            uint4 kbr[RH];
#pragma unroll
            for (int r = 0; r < RH; ++r) kbr[r] = in_kb(raw, u, r);
            float kv[8];
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {  // feature pairs (2 w2, 2 w2 + 1)
                kv[2 * w2] = kv[2 * w2 + 1] = 0.f;
#pragma unroll
                for (int rp = 0; rp < RH / 2; ++rp) {  // rank pairs (2 rp, 2 rp + 1)
                    const uint32_t a = gw[(kv0 >> 1) + rp];
                    const uint32_t b0 = (&kbr[2 * rp].x)[w2], b1 = (&kbr[2 * rp + 1].x)[w2];
                    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x05040100u);  // (b0[d], b1[d])
                    const uint32_t hi2 = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // (b0[d+1], b1[d+1])
                    kv[2 * w2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(lo), kv[2 * w2], false);
                    kv[2 * w2 + 1] =
                        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(hi2), kv[2 * w2 + 1], false);
                }
            }
            uint4 packed = make_uint4(pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3]), pack_bf16x2(kv[4], kv[5]),
                                      pack_bf16x2(kv[6], kv[7]));
            if (kPartial && key0 + k >= n_keys) packed = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(&dK[k * SKS + 8 * c8]) = packed;
        }
        // -- V^T columns: a 16-byte chunk holds 8 factor rows (whole tokens) of feature vd
        const int kbase = vbi * TOK;  // tile-relative key of the block's first token
        constexpr int TPH = 4 / RH;  // tokens in each 4-row half of a chunk
#pragma unroll
        for (int u = 0; u < V_ITEMS; ++u) {
            const int vd = 16 * (vmv0 + u) + (vcl & 15);  // the feature this chunk holds
            const uint4 vxu = in_vx(raw, u);
            const uint32_t xw[4] = {vxu.x, vxu.y, vxu.z, vxu.w};
            float v_one[2];  // RH == 4: the one token of each half, packed together below
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                // rows 16 m + 4 vg4 + 0..3 of the block: TPH whole tokens
                const uint2 vgm = in_vg(raw, m);
                const uint32_t gw[2] = {vgm.x, vgm.y};
                if constexpr (kGate) {
                    // four tokens' B_V values as cached (zero past n_keys), and their gates, written by the
                    // threads of feature 0
                    const int t0 = kbase + 16 * m + 4 * vg4;  // tile key of the first of the four
                    uint32_t x2[2] = {xw[2 * m], xw[2 * m + 1]};
#pragma unroll
                    for (int tl = 0; tl < 4; ++tl) {
                        const bool dead = kPartial && key0 + t0 + tl >= n_keys;
                        if (dead) x2[tl >> 1] &= (tl & 1) ? 0x0000ffffu : 0xffff0000u;
                        if (u == 0 && vmv0 == 0 && (vcl & 15) == 0) {
                            const uint32_t a = (tl & 1) ? (gw[tl >> 1] >> 16) : (gw[tl >> 1] & 0xffffu);
                            lds.gv[buf][t0 + tl] = dead ? 0.f : __builtin_bit_cast(float, a << 16);
                        }
                    }
                    *reinterpret_cast<uint2 *>(&dV[vd * SVS + vpos(t0)]) = make_uint2(x2[0], x2[1]);
                    continue;
                }
                float vt[TPH];
#pragma unroll
                for (int tl = 0; tl < TPH; ++tl) {
                    float acc = 0.f;
#pragma unroll
                    for (int rp = 0; rp < RH / 2; ++rp)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(gw[(tl * RH) / 2 + rp]),
                                                              as_bf16x2(xw[2 * m + (tl * RH) / 2 + rp]), acc, false);
                    vt[tl] = acc;
                    if (kPartial && key0 + kbase + (16 * m + 4 * vg4) / RH + tl >= n_keys) vt[tl] = 0.f;
                }
                uint16_t *dst = &dV[vd * SVS + vpos(kbase + (16 * m + 4 * vg4) / RH)];
                if constexpr (TPH == 4) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(vt[0], vt[1]), pack_bf16x2(vt[2], vt[3]));
                } else if constexpr (TPH == 2) {
                    *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(vt[0], vt[1]);
                } else {
                    v_one[m] = vt[0];
                }
            }
            if constexpr (TPH == 1) {
                const uint32_t pk = pack_bf16x2(v_one[0], v_one[1]);
                dV[vd * SVS + vpos(kbase + vg4)] = uint16_t(pk & 0xffffu);
                dV[vd * SVS + vpos(kbase + 4 + vg4)] = uint16_t(pk >> 16);
            }
        }
    };

    // Q operand (B of S^T): lane supplies Q~[jq][16 ks + 8 hi + e]
    bf16x8 qf[KS];
    if constexpr (kFQ) {
        factored_query_row<KS>(p, b, jq, head, hi, ctx + jq, qf);
    } else {
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
    // raw scores (the scale goes inside the exponent); lazy reference max as in decode
    const float sm = p.score_mul, lazy_raw = kLazyPrefill / sm;
    float run_m = -INFINITY, neg_ms = INFINITY, run_l = 0.f;
    const int wave_last = min(p.chunk - 1, jw + 31);
    const int jq_vis = jq < p.chunk ? ctx + jq : -1;  // last key this lane's query sees (-1: none)

    const bf16x2 ones2 = as_bf16x2(0x3F803F80u);  // (1, 1) in bf16
    auto rebuild_tile = [&](Raw &raw, int kt, int buf) {
        if (kt * kKT + kKT <= n_keys)
            rebuild(raw, kt, buf, std::false_type{});
        else
            rebuild(raw, kt, buf, std::true_type{});
    };

    // Software pipeline, one barrier per tile: the loads of tile t+1 are issued in two halves between
    // the matrix-core instructions of tile t (so the waves do not stall on a full memory queue before
    // their first MFMA), then the waves rebuild tile t+1 into the other LDS buffer.  The last iteration
    // reloads the last tile (in bounds, unused) so that the loads need no branch.  Every wave runs every
    // tile: a tile past a wave's diagonal (or a wave past the chunk's end) is fully masked, its P is
    // zero, and skipping it would put the loads behind a branch, which costs more registers than the
    // few masked tiles cost matrix-core time.
    Raw raw;
    fetch_k(raw, 0);
    fetch_v(raw, 0);
    rebuild_tile(raw, 0, 0);
    if (late) {  // a late wave runs one tile further ahead with its loads
        fetch_k(raw, min(1, n_kt - 1));
        fetch_v(raw, min(1, n_kt - 1));
    }
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (late && kt + 1 < n_kt) rebuild_tile(raw, kt + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);  // the next loads stay below the rebuild that frees their registers
        const int kn = min(kt + 1 + int(late), n_kt - 1);  // tile whose loads are issued now
        const int key0 = kt * kKT;
        // the matrix-core phase runs at a higher wave priority than the rebuild, so when both waves of a
        // SIMD can issue, the one feeding the matrix cores goes first
        __builtin_amdgcn_s_setprio(3);
        {
            const uint16_t *cK = sK[buf];
            const uint16_t *cV = sV[buf];
            // ---- S^T = K~ Q~^T for two 32-key blocks, with the K~ inputs of the next tile issued
            floatx16 s[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int v = 0; v < 16; ++v) s[kb2][v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cK[(32 * kb2 + col) * SKS + 16 * ks + 8 * hi]);
                    s[kb2] = mma32(a, qf[ks], s[kb2]);
                }
            fetch_k(raw, kn);
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global loads
            }
            if constexpr (kGate) {  // score of key k: (q . B~_K[k]) A_K[k], in fp32
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 a = *reinterpret_cast<const float4 *>(&lds.gk[buf][32 * kb2 + 8 * g + 4 * hi]);
                        s[kb2][4 * g] *= a.x;
                        s[kb2][4 * g + 1] *= a.y;
                        s[kb2][4 * g + 2] *= a.z;
                        s[kb2][4 * g + 3] *= a.w;
                    }
            }
            // ---- causal mask only where the tile crosses the diagonal (or past the chunk's end)
            if (key0 + kKT - 1 > ctx + jw || wave_last < jw + 31) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = key0 + 32 * kb2 + 8 * (v >> 2) + 4 * hi + (v & 3);
                        s[kb2][v] = key <= jq_vis ? s[kb2][v] : -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb2][v]);
            if (__any(mx > run_m + lazy_raw)) {
                const float mn = fmaxf(run_m, fmaxf(mx, __shfl_xor(mx, 32, kWave)));
                if (mn != -INFINITY) {
                    const float alpha = __builtin_amdgcn_exp2f((run_m - mn) * sm);
                    run_m = mn;
                    neg_ms = -mn * sm;
                    run_l *= alpha;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
                }
            }
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int v = 0; v < 16; ++v) s[kb2][v] = __builtin_amdgcn_exp2f(fmaf(s[kb2][v], sm, neg_ms));
            if constexpr (kGate) {  // row sum of p in fp32, then the weights p A_V[k] in place
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 a = *reinterpret_cast<const float4 *>(&lds.gv[buf][32 * kb2 + 8 * g + 4 * hi]);
                        run_l += (s[kb2][4 * g] + s[kb2][4 * g + 1]) + (s[kb2][4 * g + 2] + s[kb2][4 * g + 3]);
                        s[kb2][4 * g] *= a.x;
                        s[kb2][4 * g + 1] *= a.y;
                        s[kb2][4 * g + 2] *= a.z;
                        s[kb2][4 * g + 3] *= a.w;
                    }
            }
            // ---- O^T += V^T P^T over four 16-key steps, with the V inputs of the next tile issued; the
            // row sum takes the same bf16-rounded P the matrix cores use, two values per v_dot2 against (1, 1)
#pragma unroll
            for (int ks4 = 0; ks4 < 4; ++ks4) {
                const floatx16 &sv = s[ks4 >> 1];
                const int o8 = 8 * (ks4 & 1);
                if constexpr (kGate) {
                    // the fp32 weights as a bf16 pair hi + lo, two products with the same V^T operand: each
                    // weight reaches the accumulator to ~2^-17 of itself
                    uint32_t ph[4], pl[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float w0 = sv[o8 + 2 * i], w1 = sv[o8 + 2 * i + 1];
                        ph[i] = pack_bf16x2(w0, w1);
                        pl[i] = pack_bf16x2(w0 - __builtin_bit_cast(float, ph[i] << 16),
                                            w1 - __builtin_bit_cast(float, ph[i] & 0xffff0000u));
                    }
                    const bf16x8 pfh = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
                    const bf16x8 pfl = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cV[(32 * mb + col) * SVS + 16 * ks4 + 8 * hi]);
                        acc[mb] = mma32(a, pfh, acc[mb]);
                        acc[mb] = mma32(a, pfl, acc[mb]);
                    }
                    continue;
                }
                const uint32_t pw[4] = {pack_bf16x2(sv[o8], sv[o8 + 1]), pack_bf16x2(sv[o8 + 2], sv[o8 + 3]),
                                        pack_bf16x2(sv[o8 + 4], sv[o8 + 5]), pack_bf16x2(sv[o8 + 6], sv[o8 + 7])};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    run_l = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[i]), ones2, run_l, false);
                const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cV[(32 * mb + col) * SVS + 16 * ks4 + 8 * hi]);
                    acc[mb] = mma32(a, pf, acc[mb]);
                }
            }
            fetch_v(raw, kn);
#pragma unroll
            for (int i = 0; i < 4 * MB / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global loads
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if (!late && kt + 1 < n_kt) rebuild_tile(raw, kt + 1, buf ^ 1);
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

// Waves w and w + 4 share a SIMD.  Both run, per 64-key tile, two matrix-core phases (S, PV) and two
// vector phases (softmax, rebuild of the next tile); the second wave of each SIMD takes its rebuild at
// the top of the iteration, so the pair alternates (matrix cores | vector ALU) instead of contending for
// the same unit in step.  One barrier per tile still orders it: every wave's share of tile t+1 is written
// between the barriers that bracket iteration t, into the buffer nobody reads during iteration t.  Each
// half is its own instantiation so the register allocator sees one loop shape at a time.
template <int HP, int DP, int RH, bool kFQ, bool kF8>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) PrefillLds<DP, RH == 1> lds;
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kPrefillWaves / 2)
        prefill_body<HP, DP, RH, kFQ, true, kF8>(p, lds);
    else
        prefill_body<HP, DP, RH, kFQ, false, kF8>(p, lds);
}

// ===================================================================================================
// Wide form (bf16 cache, d_h = 128, rank 2 or 4, chunks of more than 256 rows): a work-group owns 512 query rows of
// one head, so each (key, head) pair is rebuilt once per 512 rows and the factor bytes a work-group
// loads per query row halve.  8 waves x 64 rows: each wave holds two 32-row blocks, w and 15 - w of the
// tile, so every wave has the same causal extent; 32-key tiles.  The factor pieces a wave rebuilds from
// are fetched straight into a wave-private LDS staging area (global_load_lds), so they hold no
// registers in flight, and each wave only reads back pieces it fetched itself, so the staging needs no
// barrier, only the wave's own vmcnt wait.  The ping-pong of the two waves of a SIMD is kept.
constexpr int kW2Rows = 64;                        // query rows per wave
constexpr int kQT2 = kW2Rows * kPrefillWaves;      // query rows per work-group
constexpr int kKT2 = 32;                           // keys per tile

template <int DP, int RH>
struct Prefill2Lds {
    static constexpr int TOK = kRows / RH;
    static constexpr int BPT = kKT2 / TOK;                   // cache blocks per tile
    static constexpr int MVG = kPrefillWaves / BPT;          // waves sharing one block's value chunks
    static constexpr int V_ITEMS = (DP / 16) / MVG;          // value chunks per lane
    static constexpr int K_STRIDE = 1024 + 16;               // K~ pieces, each one bank group after the last
    static constexpr int V_OFF = RH * K_STRIDE;              // then the value chunks
    static constexpr int GATE_OFF = V_OFF + V_ITEMS * 1024;  // then 3 gate slots (12 bytes used of 16 per lane)
    static constexpr int RAW_BYTES = GATE_OFF + 3 * 1024;
    uint16_t k[2][kKT2 * (DP + 8)];
    uint16_t v[2][DP * (kKT2 + 8)];
    char raw[kPrefillWaves][RAW_BYTES];
};

typedef __attribute__((address_space(3))) void *lds_ptr;

template <int HP, int DP, int RH, bool kFQ, bool late>
__device__ __forceinline__ void prefill2_body(const PrefillParams &p, Prefill2Lds<DP, RH> &lds) {
    using LD = Prefill2Lds<DP, RH>;
    constexpr int KS = DP / 16;
    constexpr int MB = DP / 32;
    constexpr int NB = HP / 16;
    constexpr int KBS = DP / 32;
    constexpr int TOK = LD::TOK, BPT = LD::BPT, MVG = LD::MVG, V_ITEMS = LD::V_ITEMS;
    constexpr int SKS = DP + 8;
    constexpr int SVS = kKT2 + 8;
    constexpr int BLK = 2 * kRows * (HP + DP);
    constexpr int OFF_AV = kRows * HP, OFF_BK = 2 * kRows * HP, OFF_BV = 2 * kRows * HP + kRows * DP;
    constexpr int C8 = DP / 8;
    static_assert(RH >= 2, "rank 1 takes the 256-row form, which keeps its gates in fp32");
    static_assert(kKT2 * C8 == kPrefillThreads, "one K~ item per thread");
    static_assert(MVG * BPT == kPrefillWaves && V_ITEMS * MVG == DP / 16, "V items must tile the group");

    const int n_qt = (p.chunk + kQT2 - 1) / kQT2;
    const int L = blockIdx.x;
    int b, head, qt;
    if (p.batch % kXcds == 0) {
        const int per_seq = p.h * n_qt;
        b = L % kXcds + kXcds * (L / (kXcds * per_seq));
        const int r = (L / kXcds) % per_seq;
        head = r / n_qt;
        qt = r % n_qt;
    } else {
        qt = L % n_qt;
        head = (L / n_qt) % p.h;
        b = L / (n_qt * p.h);
    }
    const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hi = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j0 = qt * kQT2;
    const int jw[2] = {j0 + 32 * w, j0 + 32 * (2 * kPrefillWaves - 1 - w)};  // the wave's two row blocks
    const int jq[2] = {jw[0] + col, jw[1] + col};
    int ctx = p.ctx_len[b];
    const int64_t start = p.seq_start[b];
    ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
    float *out = p.out + int64_t(b) * p.chunk * p.h * p.d_h;

    if (seq_rejected(start, int64_t(ctx) + p.chunk, TOK, p.capacity)) {  // as in the 256-row form
        for (int idx = tid; idx < kQT2 * p.d_h; idx += kPrefillThreads) {
            const int j = j0 + idx / p.d_h, d = idx % p.d_h;
            if (j < p.chunk) out[(int64_t(j) * p.h + head) * p.d_h + d] = __builtin_nanf("");
        }
        return;
    }
    const char *seq = reinterpret_cast<const char *>(p.cache) + (start / TOK) * int64_t(BLK) * 2;
    const int j_last = min(p.chunk, j0 + kQT2) - 1;
    const int n_keys = ctx + j_last + 1;
    const int n_kt = (n_keys + kKT2 - 1) / kKT2;
    const int gate_lane = head & 15, gate_nb = head >> 4;

    // ---- this lane's pieces.  K~: wave w owns one 16-row group of the tile's factor rows (16 / RH keys)
    // over RH of the 4 32-feature column blocks, so each of its RH fetches is one whole, contiguous 1 KB
    // piece of the cache block; lane (key kl, chunk) then reads the RH rank pieces of its key from the
    // staging area.  V: V_ITEMS contiguous value chunks of one cache block.
    // A K~ piece's 64 chunks are (sub, row): features 8 sub .. 8 sub + 7 of factor row `row` of the group, at
    // chunk 16 sub + row of the cache block.  Staged in that order, the 16 lanes that read one rank at a time
    // (rank 4: one key over four pieces and four subs; rank 2: two keys over two pieces and four subs) would hit
    // chunks that are multiples of 256 bytes apart, i.e. the same four LDS banks or two groups of them.  So
    // chunk (sub, row) goes to slot 16 sub + (row ^ 4 sub) (the rows of a sub stay in its 256 bytes), and
    // piece q starts 16 q bytes past a 1 KB boundary: the 16 lanes' reads then fall in 16 different bank groups.
    constexpr int WPG = 4 / RH;                       // waves per 16-row group
    const int gi = w / WPG;                           // the wave's 16-row group inside the tile
    const int kbw0 = (w % WPG) * RH;                  // its first 32-feature column block
    const int kl = lane / (4 * RH);                   // this lane's key inside the group
    const int k_blk = gi / 2, k_mb = gi % 2;          // cache block (tile-relative) and row group in it
    const int lane_sw = lane ^ ((lane >> 4) << 2);   // the cache chunk this lane stages into its slot
    const uint32_t k_off_b = uint32_t(k_blk * BLK + OFF_BK + ((k_mb * KBS + kbw0) * kWave + lane_sw) * 8) * 2u;
    const int k_gl = 16 * ((kl * RH) >> 2) + gate_lane;
    const uint32_t k_off_gate = uint32_t(k_blk * BLK + ((k_mb * NB + gate_nb) * kWave + k_gl) * 4) * 2u;
    const int vrow = w, vcl = lane, vg4 = vcl >> 4;
    const int vbi = vrow % BPT, vmv0 = (vrow / BPT) * V_ITEMS;
    const uint32_t v_off = uint32_t(vbi * BLK + OFF_BV + (vmv0 * kWave + vcl) * 8) * 2u;
    const int v_gl = 16 * vg4 + gate_lane;
    const uint32_t v_off_gate = uint32_t(vbi * BLK + OFF_AV + (gate_nb * kWave + v_gl) * 4) * 2u;

    char *rw = lds.raw[w];
    auto tile_base = [&](int kt) { return seq + int64_t((kt * kKT2) / TOK) * BLK * 2; };
    auto tile_last_blk = [&](int kt) {
        const int key0 = kt * kKT2;
        return key0 + kKT2 <= n_keys ? 1 << 20 : (n_keys - 1) / TOK - key0 / TOK;
    };
    // Fetch of one tile's pieces into the wave's staging area (the 8-byte gate pieces as 12-byte
    // transfers, which land 16 bytes apart).  Blocks past the last live one are replaced by it.
    auto fetch = [&](int kt) {
        const char *tb = tile_base(kt);
        const int last_blk = tile_last_blk(kt);
        // the per-lane offsets are rebuilt here (opaque to the optimizer) rather than kept live per piece
        uint32_t ko = k_off_b + uint32_t((min(k_blk, last_blk) - k_blk) * BLK) * 2u;
        uint32_t kg = k_off_gate - k_off_b;
        uint32_t vo = v_off + uint32_t((min(vbi, last_blk) - vbi) * BLK) * 2u;
        uint32_t vg = v_off_gate - v_off;
        asm volatile("" : "+v"(ko), "+v"(kg), "+v"(vo), "+v"(vg));
#pragma unroll
        for (int q = 0; q < RH; ++q)
            __builtin_amdgcn_global_load_lds(tb + uint32_t(ko + q * kWave * 16), (lds_ptr)(rw + q * LD::K_STRIDE), 16,
                                             0, 0);
        __builtin_amdgcn_global_load_lds(tb + uint32_t(ko + kg), (lds_ptr)(rw + LD::GATE_OFF), 12, 0, 0);
#pragma unroll
        for (int u = 0; u < V_ITEMS; ++u)
            __builtin_amdgcn_global_load_lds(tb + uint32_t(vo + u * kWave * 16), (lds_ptr)(rw + LD::V_OFF + u * 1024), 16,
                                             0, 0);
#pragma unroll
        for (int m = 0; m < 2; ++m)
            __builtin_amdgcn_global_load_lds(tb + uint32_t(vo + vg + m * NB * kWave * 8),
                                             (lds_ptr)(rw + LD::GATE_OFF + (1 + m) * 1024), 12, 0, 0);
    };
    // The rebuild: bf16 pair products with fp32 accumulation, one bf16 rounding.
    // Its per-lane addresses are derived from an opaque copy of the lane index, so they live only here.
    auto rebuild = [&](int kt, int buf, auto partial_tag) {
        constexpr bool kPartial = decltype(partial_tag)::value;
        uint32_t ln = lane;  // unsigned: the divisions and remainders below are shifts and masks
        asm volatile("" : "+v"(ln));
        __builtin_assume(ln < 64u);  // and the products below fit 24-bit multiplies
        const int key0 = kt * kKT2;
        const char *rl = rw + 16 * ln;  // this lane's 16-byte slot of each staged piece
        const uint32_t kl_ = ln / (4 * RH), cl_ = ln % (4 * RH);
        const int kb_ = kbw0 + int(cl_ / 4), sub_ = int(cl_ % 4);
        const int kk_ = (16 * gi) / RH + int(kl_);
        const int kv0_ = int(kl_ * RH) & 3;
        {
            const uint32_t *gp = reinterpret_cast<const uint32_t *>(rl + LD::GATE_OFF);
            const uint32_t gw[2] = {gp[0], gp[1]};
            // rank pieces of this lane's key: row kl RH + r of sub `sub` in piece kb - kbw0, in slot
            // 16 sub + ((kl RH) ^ 4 sub) + r (r only occupies the row's low bits)
            const char *kp = rw + (kb_ - kbw0) * LD::K_STRIDE + 16 * (16 * sub_ + (int(kl_ * RH) ^ (4 * sub_)));
            uint4 kbr[RH];
#pragma unroll
            for (int r = 0; r < RH; ++r) kbr[r] = *reinterpret_cast<const uint4 *>(kp + 16 * r);
            float kv[8];
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {  // feature pairs (2 w2, 2 w2 + 1)
                kv[2 * w2] = kv[2 * w2 + 1] = 0.f;
#pragma unroll
                for (int rp = 0; rp < RH / 2; ++rp) {  // rank pairs (2 rp, 2 rp + 1)
                    const uint32_t a = gw[(kv0_ >> 1) + rp];
                    const uint32_t b0 = (&kbr[2 * rp].x)[w2], b1 = (&kbr[2 * rp + 1].x)[w2];
                    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x05040100u);
                    const uint32_t hi2 = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
                    kv[2 * w2] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(lo), kv[2 * w2], false);
                    kv[2 * w2 + 1] =
                        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(hi2), kv[2 * w2 + 1], false);
                }
            }
            uint4 packed = make_uint4(pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3]), pack_bf16x2(kv[4], kv[5]),
                                      pack_bf16x2(kv[6], kv[7]));
            if (kPartial && key0 + kk_ >= n_keys) packed = make_uint4(0, 0, 0, 0);
            const uint32_t k_at = uint32_t(kk_) * SKS + uint32_t(32 * kb_ + 8 * sub_);  // 32-bit LDS index math
            *reinterpret_cast<uint4 *>(&lds.k[buf][k_at]) = packed;
        }
        __builtin_amdgcn_sched_barrier(0);
        const int vg4_ = int(ln >> 4);
        const int kbase = vbi * TOK;
        constexpr int TPH = 4 / RH;
        uint32_t gv[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint32_t *gp = reinterpret_cast<const uint32_t *>(rl + LD::GATE_OFF + (1 + m) * 1024);
            gv[m][0] = gp[0];
            gv[m][1] = gp[1];
        }
        uint16_t *dV = &lds.v[buf][uint32_t(16 * vmv0 * SVS) + (ln & 15u) * SVS];
#pragma unroll
        for (int u = 0; u < V_ITEMS; ++u) {
            const uint4 vxu = *reinterpret_cast<const uint4 *>(rl + LD::V_OFF + u * 1024);
            const uint32_t xw[4] = {vxu.x, vxu.y, vxu.z, vxu.w};
            float v_one[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float vt[TPH];
#pragma unroll
                for (int tl = 0; tl < TPH; ++tl) {
                    float acc = 0.f;
#pragma unroll
                    for (int rp = 0; rp < RH / 2; ++rp)
                        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(gv[m][(tl * RH) / 2 + rp]),
                                                              as_bf16x2(xw[2 * m + (tl * RH) / 2 + rp]), acc, false);
                    vt[tl] = acc;
                    if (kPartial && key0 + kbase + (16 * m + 4 * vg4_) / RH + tl >= n_keys) vt[tl] = 0.f;
                }
                uint16_t *dst = dV + 16 * u * SVS + vpos(kbase + (16 * m + 4 * vg4_) / RH);
                if constexpr (TPH == 4) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(vt[0], vt[1]), pack_bf16x2(vt[2], vt[3]));
                } else if constexpr (TPH == 2) {
                    *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(vt[0], vt[1]);
                } else {
                    v_one[m] = vt[0];
                }
            }
            if constexpr (TPH == 1) {
                const uint32_t pk = pack_bf16x2(v_one[0], v_one[1]);
                dV[16 * u * SVS + vpos(kbase + vg4_)] = uint16_t(pk & 0xffffu);
                dV[16 * u * SVS + vpos(kbase + 4 + vg4_)] = uint16_t(pk >> 16);
            }
        }
    };
    auto rebuild_tile = [&](int kt, int buf) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's staged pieces have landed
        if (kt * kKT2 + kKT2 <= n_keys)
            rebuild(kt, buf, std::false_type{});
        else
            rebuild(kt, buf, std::true_type{});
    };

    // Q operands of the two row blocks
    bf16x8 qf[2][KS];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        if constexpr (kFQ) {
            factored_query_row<KS>(p, b, jq[nb], head, hi, ctx + jq[nb], qf[nb]);
        } else {
            const uint16_t *qrow = reinterpret_cast<const uint16_t *>(p.q) +
                                   (int64_t(b) * p.chunk + jq[nb]) * p.h * p.d_h + int64_t(head) * p.d_h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = 16 * ks + 8 * hi;
                qf[nb][ks] = jq[nb] < p.chunk ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + d0))
                                              : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
            }
        }
    }

    floatx16 acc[2][MB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[nb][mb][v] = 0.f;
    const float sm = p.score_mul, lazy_raw = kLazyPrefill / sm;
    float run_m[2] = {-INFINITY, -INFINITY}, neg_ms[2] = {INFINITY, INFINITY}, run_l[2] = {0.f, 0.f};
    int wave_last[2], jq_vis[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        wave_last[nb] = min(p.chunk - 1, jw[nb] + 31);
        jq_vis[nb] = jq[nb] < p.chunk ? ctx + jq[nb] : -1;
    }
    const bf16x2 ones2 = as_bf16x2(0x3F803F80u);

    // The pieces of the tile a wave rebuilds next are fetched while it runs the matrix-core
    // instructions of the current tile (interleaved with the first row block's score products).
    fetch(0);
    rebuild_tile(0, 0);
    if (late) fetch(min(1, n_kt - 1));
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (late && kt + 1 < n_kt) rebuild_tile(kt + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        const int kf = min(kt + 1 + int(late), n_kt - 1);  // tile whose pieces are fetched now
        const int key0 = kt * kKT2;
        // the matrix-core phase runs at a higher wave priority than the rebuild, so when both waves of a
        // SIMD can issue, the one feeding the matrix cores goes first
        __builtin_amdgcn_s_setprio(3);
        {
            const uint16_t *cK = lds.k[buf];
            const uint16_t *cV = lds.v[buf];
            // the two row blocks one after the other (one score tile live at a time): the later block
            // first (it carries the fetches), then the earlier one, skipped once its rows see no key
            // of the tile
#pragma unroll
            for (int nbi = 0; nbi < 2; ++nbi) {
                const int nb = 1 - nbi;
                __builtin_amdgcn_sched_barrier(0);
                if (nb == 0 && key0 > ctx + wave_last[0]) continue;
                floatx16 s;
#pragma unroll
                for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cK[col * SKS + 16 * ks + 8 * hi]);
                    s = mma32(a, qf[nb][ks], s);
                }
                if (nb == 1) {
                    fetch(kf);
                    // operand reads two ahead of the matrix cores, the fetches between them
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                    for (int i = 0; i < KS - 2; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                    for (int i = 0; i < KS - 2; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                if (key0 + kKT2 - 1 > ctx + jw[nb] || wave_last[nb] < jw[nb] + 31) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = key0 + 8 * (v >> 2) + 4 * hi + (v & 3);
                        s[v] = key <= jq_vis[nb] ? s[v] : -INFINITY;
                    }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
                if (__any(mx > run_m[nb] + lazy_raw)) {
                    const float mn = fmaxf(run_m[nb], fmaxf(mx, __shfl_xor(mx, 32, kWave)));
                    if (mn != -INFINITY) {
                        const float alpha = __builtin_amdgcn_exp2f((run_m[nb] - mn) * sm);
                        run_m[nb] = mn;
                        neg_ms[nb] = -mn * sm;
                        run_l[nb] *= alpha;
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] *= alpha;
                    }
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) s[v] = __builtin_amdgcn_exp2f(fmaf(s[v], sm, neg_ms[nb]));
#pragma unroll
                for (int ks4 = 0; ks4 < 2; ++ks4) {
                    const int o8 = 8 * ks4;
                    const uint32_t pw[4] = {pack_bf16x2(s[o8], s[o8 + 1]), pack_bf16x2(s[o8 + 2], s[o8 + 3]),
                                            pack_bf16x2(s[o8 + 4], s[o8 + 5]), pack_bf16x2(s[o8 + 6], s[o8 + 7])};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        run_l[nb] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[i]), ones2, run_l[nb], false);
                    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&cV[(32 * mb + col) * SVS + 16 * ks4 + 8 * hi]);
                        acc[nb][mb] = mma32(a, pf, acc[nb][mb]);
                    }
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if (!late && kt + 1 < n_kt) rebuild_tile(kt + 1, buf ^ 1);
        __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the last (unused) fetches have landed

#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const float l = run_l[nb] + __shfl_xor(run_l[nb], 32, kWave);
        if (jq[nb] < p.chunk) {
            const float inv = p.out_mul / l;
            float *o = out + (int64_t(jq[nb]) * p.h + head) * p.d_h;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int d = 32 * mb + 8 * v4 + 4 * hi;
                    *reinterpret_cast<float4 *>(o + d) =
                        make_float4(acc[nb][mb][4 * v4] * inv, acc[nb][mb][4 * v4 + 1] * inv, acc[nb][mb][4 * v4 + 2] * inv,
                                    acc[nb][mb][4 * v4 + 3] * inv);
                }
        }
    }
}

template <int HP, int DP, int RH, bool kFQ>
__global__ __launch_bounds__(kPrefillThreads) void prefill2_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) Prefill2Lds<DP, RH> lds;
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= kPrefillWaves / 2)
        prefill2_body<HP, DP, RH, kFQ, true>(p, lds);
    else
        prefill2_body<HP, DP, RH, kFQ, false>(p, lds);
}

// The wide form pays off once a chunk fills more than one 256-row work-group.  Rank 1 stays on the
// 256-row form, whose rebuild is a copy at that rank: the fp32 gates do not fit the wide form's registers.
bool use_wide(const PrefillParams &p) { return p.d_h == 128 && p.chunk > kQT; }

template <int HP, int DP, int RH, bool kF8>
hipError_t launch_one(const PrefillParams &p, hipStream_t s) {
    if constexpr (DP == 128 && !kF8 && RH >= 2) {
        if (use_wide(p)) {
            const dim3 grid2(unsigned(((p.chunk + kQT2 - 1) / kQT2) * p.h * p.batch));
            if (p.r_q > 0)
                hipLaunchKernelGGL((prefill2_kernel<HP, DP, RH, true>), grid2, dim3(kPrefillThreads), 0, s, p);
            else
                hipLaunchKernelGGL((prefill2_kernel<HP, DP, RH, false>), grid2, dim3(kPrefillThreads), 0, s, p);
            return hipGetLastError();
        }
    }
    const dim3 grid(unsigned(((p.chunk + kQT - 1) / kQT) * p.h * p.batch));
    if (p.r_q > 0)
        hipLaunchKernelGGL((prefill_kernel<HP, DP, RH, true, kF8>), grid, dim3(kPrefillThreads), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_kernel<HP, DP, RH, false, kF8>), grid, dim3(kPrefillThreads), 0, s, p);
    return hipGetLastError();
}

template <int HP, int DP, bool kF8>
hipError_t launch_rank(int RH, const PrefillParams &p, hipStream_t s) {
    switch (RH) {
        case 1: return launch_one<HP, DP, 1, kF8>(p, s);
        case 2: return launch_one<HP, DP, 2, kF8>(p, s);
        case 4: return launch_one<HP, DP, 4, kF8>(p, s);
    }
    return hipErrorInvalidValue;
}

// (the padded (heads, head dim) pairs the cache layer supports with bf16 operands)
#define TPA_PREFILL_SHAPES(X) X(16, 64) X(16, 128) X(32, 64) X(32, 128) X(64, 64)

}  // namespace

// bf16 operands: a bf16 cache, or an E4M3 cache (decoded to bf16 in the rebuild)
bool prefill_supported(const Layout &L) {
    if (L.es != 2 && !L.f8) return false;
#define X(HP_, DP_) \
    if (L.HP == HP_ && L.DP == DP_) return true;
    TPA_PREFILL_SHAPES(X)
#undef X
    return false;
}

int prefill_rows_per_group(const Layout &L, const PrefillParams &p) {
    return L.DP == 128 && !L.f8 && L.RH >= 2 && use_wide(p) ? kQT2 : kQT;
}

hipError_t launch_prefill(const Layout &L, const PrefillParams &p, hipStream_t s) {
#define X(HP_, DP_)                                                                   \
    if (L.f8 && L.HP == HP_ && L.DP == DP_) return launch_rank<HP_, DP_, true>(L.RH, p, s); \
    if (L.es == 2 && L.HP == HP_ && L.DP == DP_) return launch_rank<HP_, DP_, false>(L.RH, p, s);
    TPA_PREFILL_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace tpa
