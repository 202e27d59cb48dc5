// Internal definitions shared by the libtpa kernels and the C ABI layer.
//
// Cache block layout.  A block holds kRows = 32 factor rows; a row is one
// (token, rank) pair and a token owns RH consecutive rows, where RH is the
// rank padded to 1, 2 or 4 (rows r >= R_K or r >= R_V are stored as zeros).
// A block therefore holds 32 / RH tokens.  Heads are padded to HP (a
// multiple of 16) and the head dimension to DP; padding is stored as zeros.
//
// The decode kernel runs two matrix-core contractions per block with the
// 16x16 MFMA shapes (bf16 16x16x32: E = 8 k-values per lane; fp32 16x16x4:
// E = 1):
//   scores  U^T[row][head] = B~_K[row][:] . q~[head][:]   (A operand: B~_K rows)
//   values  O^T[d][head]  += B_V[:][d]^T . W[:][head]      (A operand: B_V columns)
// and applies the head factors A_K, A_V as per-(row, head) gates on the
// score accumulators.  Each region of a block is stored exactly in the
// per-lane order of the operand or accumulator it feeds, so one wave-wide
// load of 16 (or 8) bytes per lane reads a contiguous 1 KiB (512 B) span:
//   A_K, A_V gates : [mblk 2][NB][lane 64][4]     row = 16 mblk + 4 (lane/16) + v,
//                                                 head = 16 nb + lane%16
//   B~_K           : [mblk 2][KBS][lane 64][E]    row = 16 mblk + lane%16,
//                                                 d = 4E kb + E (lane/16) + e
//   B_V            : [MBV][KBV][lane 64][E]        d = 16 mv + lane%16,
//                                                 row = score row of slot t = E q + e:
//                                                 16 (t/4) + 4 (lane/16) + t%4
// so the score accumulator a lane holds (rows 4(lane/16)+v of both score
// row blocks, one head) is exactly the k-slice it must supply to the value
// contraction: no data moves between lanes between the two contractions.
//
// 8-bit factor storage (OCP E4M3 codes; bf16 queries and matrix-core
// operands): the same per-lane pieces, one byte per element, with two pieces
// paired per lane so that a lane still loads 16 (gates: 8) contiguous bytes:
//   gates : [NB][lane 64][mblk 2][4]      (both row blocks of a head block)
//   B~_K  : [KBS][lane 64][mblk 2][8]     (both row blocks of a k-block)
//   B_V   : [MBV/2][lane 64][2][8]        (value M blocks 2j and 2j+1)
// The kernels turn the codes into bf16 fragments and fp32 gates in registers;
// a stored value is code * scale with one scale per factor tensor, folded into
// the score and output multipliers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpa {

constexpr int kRows = 32;  // factor rows per cache block
constexpr int kWave = 64;
constexpr int kAppendThreads = 128;   // work-items per append / read work-group
constexpr int kPrefillThreads = 512;  // work-items per prefill work-group
constexpr int kPrefillRows = 256;     // query rows per prefill work-group (the wide form takes twice as many)
// A one-dimensional launch counts its work-items (work-groups x work-items per group) in 32 bits.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads of cache data: each byte of the cache is read once per call, so the loads are
// marked non-temporal (they do not displace reusable lines in L2 / the last-level cache); measured
// on MI355X this lifts a plain 16-byte-per-lane read stream from ~6.2 to ~7.1 TB/s.
__device__ __forceinline__ u32x4 stream_load16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 stream_load8(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

// Runtime description of one cache layout (host and device).
struct Layout {
    int HP, DP, RH, E;  // padded heads, padded head dim, padded rank, k-values per lane
    int es;             // element size in bytes
    int f8;             // 1: E4M3 codes in the paired 8-bit layout (bf16 queries)

    __host__ __device__ int tok_per_block() const { return kRows / RH; }
    __host__ __device__ int NB() const { return HP / 16; }
    __host__ __device__ int KBS() const { return DP / (4 * E); }
    __host__ __device__ int MBV() const { return DP / 16; }
    __host__ __device__ int KBV() const { return kRows / (4 * E); }
    __host__ __device__ int64_t block_elems() const { return 2LL * kRows * (HP + DP); }
    __host__ __device__ int off_ak() const { return 0; }
    __host__ __device__ int off_av() const { return kRows * HP; }
    __host__ __device__ int off_bk() const { return 2 * kRows * HP; }
    __host__ __device__ int off_bv() const { return 2 * kRows * HP + kRows * DP; }

    // element offsets inside a block region
    __host__ __device__ int gate(int row, int head) const {
        int mb = row >> 4, nb = head >> 4, lane = 16 * ((row & 15) >> 2) + (head & 15), v = row & 3;
        if (f8) return ((nb * kWave + lane) * 2 + mb) * 4 + v;
        return ((mb * NB() + nb) * kWave + lane) * 4 + v;
    }
    __host__ __device__ int bk(int row, int d) const {
        int mb = row >> 4, kb = d / (4 * E), lane = 16 * ((d % (4 * E)) / E) + (row & 15), e = d % E;
        if (f8) return ((kb * kWave + lane) * 2 + mb) * E + e;
        return ((mb * KBS() + kb) * kWave + lane) * E + e;
    }
    __host__ __device__ int bv(int row, int d) const {
        int t = 4 * (row >> 4) + (row & 3), g = (row & 15) >> 2;
        int q = t / E, e = t % E, mv = d >> 4, lane = 16 * g + (d & 15);
        if (f8) return (((mv >> 1) * kWave + lane) * 2 + (mv & 1)) * E + e;  // E = 8: q = 0
        return ((mv * KBV() + q) * kWave + lane) * E + e;
    }
};

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Padded rank: 1, 2 or 4 rows per token.
__host__ __device__ inline int padded_rank(int RK, int RV) {
    int r = RK > RV ? RK : RV;
    return r <= 1 ? 1 : (r <= 2 ? 2 : 4);
}

// fmt 1: E4M3 storage (dtype must be bf16, checked by the caller)
__host__ __device__ inline Layout make_layout(int h, int d_h, int RK, int RV, int dtype, int fmt = 0) {
    Layout L;
    L.E = dtype == 1 ? 8 : 1;
    L.es = fmt == 1 ? 1 : (dtype == 1 ? 2 : 4);
    L.f8 = fmt == 1 ? 1 : 0;
    L.HP = round_up(h, 16);
    L.DP = round_up(d_h, dtype == 1 ? 32 : 16);
    L.RH = padded_rank(RK, RV);
    return L;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// bf16 <-> fp32 (bit level; bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// ---- OCP E4M3 codes (8-bit factor storage).  The gfx950 conversions decode exactly; the encoder rounds
// to nearest even but turns magnitudes past 464 into NaN, so values are first clamped to the largest
// finite magnitude, 448 (saturation; NaN stays NaN).
__device__ __forceinline__ float e4m3_clamp(float x) { return fabsf(x) > 448.f ? copysignf(448.f, x) : x; }
// two values -> two codes in the low 16 bits (first value in the low byte)
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
    return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false)) & 0xffffu;
}
__device__ __forceinline__ uint8_t e4m3_one(float a) { return uint8_t(e4m3_pair(a, 0.f) & 0xffu); }
// four codes (bytes of w, low first) -> four fp32
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *g) {
    const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true);
    g[0] = lo.x;
    g[1] = lo.y;
    g[2] = hi.x;
    g[3] = hi.y;
}
// four codes -> two packed bf16 pairs (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}
// eight codes -> eight bf16 (an MFMA fragment's 16 bytes)
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    const uint2 a = e4m3x4_to_bf16x4(w0), b = e4m3x4_to_bf16x4(w1);
    return make_uint4(a.x, a.y, b.x, b.y);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int dtype = 0;
    __device__ static float load(const float *p, int64_t i) { return p[i]; }
    __device__ static float to_f32(float x) { return x; }
    __device__ static float from_f64(double x) { return float(x); }
};
template <>
struct Elem<uint16_t> {
    static constexpr int dtype = 1;
    __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
    __device__ static uint16_t from_f64(double x) { return f32_to_bf16_rne(float(x)); }
};

// ---- RoPE (TPA notes page, Key design, RoPE compatibility): RoFormer pairs (2j, 2j+1),
// theta_j = base^(-2j/d_h), (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a), a = pos * theta_j.
// Shared by the cache append and the fused decode step, so both write bit-identical records.

// Frequencies theta_j, j < d_h/2, computed once per call on the host in fp64 and passed by value.
struct RopeTable {
    double theta[128];
};

// Arithmetic of the rotation.  The angle pos * theta_j is always formed and reduced modulo 2 pi in
// fp64 (positions reach 131072 and beyond, where an fp32 angle is off by milliradians).  For bf16
// storage, cos/sin of the reduced angle and the rotation itself are then fp32: their error, ~1e-7
// relative, is far below half a bf16 unit, so the stored value is the correctly rounded rotation
// except within 1e-7 of a rounding tie (at most one unit off).  fp32 storage keeps fp64 throughout.
template <typename T>
struct RopeMath {
    using F = double;
    __device__ static void sincos_reduced(double r, F *s, F *c) { sincos(r, s, c); }
};
template <>
struct RopeMath<uint16_t> {
    using F = float;
    __device__ static void sincos_reduced(double r, F *s, F *c) { sincosf(float(r), s, c); }
};

// cos and sin of pos * theta into cs[0], cs[1].  The reduction is Cody-Waite with 2 pi split in two
// doubles; positions are int32, so |angle| < 2^31 and r is exact to ~1e-15 before sincos sees |r| <= pi.
template <typename T>
__device__ inline void rope_cos_sin(typename RopeMath<T>::F *cs, double pos, double theta) {
    constexpr double kTwoPiHi = 6.283185307179586232;    // nearest double to 2 pi
    constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2 pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = pos * theta;
    const double k = rint(phi * kInvTwoPi);
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, phi));
    RopeMath<T>::sincos_reduced(r, &cs[1], &cs[0]);
}

// (a, b) rotated by the angle whose cos, sin are c, s, in the precision F; the caller rounds once to T.
template <typename F>
__device__ inline void rope_rotate(F a, F b, F c, F s, F &y0, F &y1) {
    y0 = fma(a, c, -(b * s));
    y1 = fma(a, s, b * c);
}

// New token of a fused decode step (tpa_decode_step): unrotated factors [batch][R][h | d_h].
struct StepInputs {
    const void *A_K, *B_K, *A_V, *B_V;
    void *cache;       // the cache, written at slot seq_start[b] + seq_len[b]
    int64_t capacity;  // slots in the cache
    float inv_scale[4];  // E4M3 cache: code = E4M3(value * inv_scale) for A_K, B_K, A_V, B_V
};

// Parameters of one decode call, shared by the split and merge kernels.
struct DecodeParams {
    const void *cache;
    const int64_t *seq_start;
    const int32_t *seq_len;
    const void *q;  // [batch][h][d_h]
    float *out;     // [batch][h][d_h]
    float *ws_o;    // [grid + batch][HP][DP]: one partial per (work-group, sequence) job, at wg + b
    float *ws_ml;   // [grid + batch][HP][2]
    int2 *ws_meta;  // [batch]: the first and last work-group holding a piece of the sequence
    int64_t capacity;  // cache slots: a sequence reaching past them (or misaligned) gets NaN output
    int h, d_h, RK, RV;
    int batch, max_len;
    int split_blocks;  // blocks per work-group; 0: the kernel shares the batch's blocks out over the grid
    int grid;          // split work-groups
    int merge_parts;   // the planner's estimate of the pieces per sequence (picks the merge's width)
    float score_mul;  // scale * log2(e) / R_K
    float out_mul;    // 1 / R_V
    // Fused step (tpa_decode_step) when nonzero: q is unrotated and sits at position seq_len[b]; the
    // split kernel rotates it, the merge kernel folds in the new token and writes its record.
    int step;
    StepInputs st;
    RopeTable rope;
    // Factored query (tpa_decode_fq) when r_q > 0: q holds B_Q [batch][r_q][d_h] (unrotated; the built
    // query is rotated at position seq_len[b] with the rope table), a_q holds A_Q [batch][r_q][h].
    int r_q;
    const void *a_q;
};

struct PrefillParams {
    const void *cache;
    const int64_t *seq_start;
    const int32_t *ctx_len;
    const void *q;  // [batch][chunk][h][d_h]
    float *out;     // [batch][chunk][h][d_h]
    int64_t capacity;  // cache slots: a sequence reaching past them (or misaligned) gets NaN output
    int h, d_h, RK, RV;
    int batch, chunk, max_ctx;
    float score_mul;  // scale * log2(e) / R_K
    float out_mul;    // 1 / R_V
    // Factored query (tpa_prefill_chunk_fq) when r_q > 0: q holds B_Q [batch][chunk][r_q][d_h] (unrotated;
    // row j's built query is rotated at position ctx_len[b] + j with the rope table), a_q holds
    // A_Q [batch][chunk][r_q][h].
    int r_q;
    const void *a_q;
    RopeTable rope;
};

// A sequence the kernels refuse to read: its first slot is negative or not at a block boundary, or its
// slots [start, start + n_slots) reach past the cache's capacity.  Such a sequence gets NaN output and no
// slot of it is read or written (the host can only check sizes; starts and lengths live in device memory).
__host__ __device__ inline bool seq_rejected(int64_t start, int64_t n_slots, int tok_per_block, int64_t capacity) {
    return start < 0 || start % tok_per_block != 0 || start > capacity - n_slots;
}

// Host: theta_j = base^(-2j/d_h) in fp64 (zeros past d_h/2).
RopeTable make_rope_table(int d_h, double base);

// Work-groups of tpa_cache_append per query token of q_rows rows.
int64_t append_q_groups(int q_rows, int d_h);

// Launchers (return hipError_t of the launch).
hipError_t launch_append(const Layout &L, int h, int d_h, int RK, int RV, double base, void *cache,
                         int64_t capacity, int64_t n_kv, const int64_t *slot, const int32_t *kv_pos,
                         const void *A_K, const void *B_K, const void *A_V, const void *B_V, int64_t n_q,
                         int q_rows, const int32_t *q_pos, const void *q_in, void *q_out, const float *inv_scale,
                         hipStream_t s);
hipError_t launch_read(const Layout &L, int h, int d_h, int RK, int RV, const void *cache, int64_t capacity,
                       int64_t n, const int64_t *slot, void *A_K, void *B_K, void *A_V, void *B_V,
                       hipStream_t s);
bool decode_supported(const Layout &L);
hipError_t launch_decode(const Layout &L, const DecodeParams &p, hipStream_t s);
int decode_merge_threads(const Layout &L, const DecodeParams &p);  // the merge kernel's work-group size
bool prefill_supported(const Layout &L);
hipError_t launch_prefill(const Layout &L, const PrefillParams &p, hipStream_t s);
int prefill_rows_per_group(const Layout &L, const PrefillParams &p);  // query rows per prefill work-group

}  // namespace tpa
