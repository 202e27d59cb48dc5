// C ABI of libtpa: argument checks, launch planning and dispatch.
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect and the checks work on a machine without a GPU.
#include <math.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/tpa.h"
#include "common.h"

// tpa_decode_noalloc keeps the pieces' partials and range records (the workspace of tpa_decode) in this
// array instead of a caller's buffer.  Each GPU the library runs on holds its own copy until the process
// ends; in host code the name is only a stand-in, so its device address is looked up per device
// (scratch_address below) and only that address is ever passed on.
constexpr int64_t kScratchBytes = TPA_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using tpa::Layout;

// Decode work partition: the split kernel shares the batch's blocks out evenly over its work-groups (it
// scans the device-resident lengths itself), so the host only picks the grid: at most one work-group per
// compute unit of an MI355X (256), and for the wide layouts (HP * DP >= 2048, whose waves need most of
// the register file) 192 of them, which measured faster on the ragged 128-sequence workload (831 vs 851
// us) and leaves a quarter of the CUs to work on another stream; never more than pieces of 16 blocks
// would fill.  A caller's split_tokens fixes the blocks per work-group instead, and the grid is sized for
// the longest batch the arguments allow.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kWideDecodeGroups = 192;
constexpr int kDecodeWaves = 4;

bool dims_valid(const tpa_dims *d) {
    if (!d) return false;
    if (d->h < 1 || d->h > 64) return false;
    if (d->d_h < 2 || d->d_h > 256 || (d->d_h & 1)) return false;
    if (d->R_K < 1 || d->R_K > 4 || d->R_V < 1 || d->R_V > 4) return false;
    if (d->dtype != TPA_F32 && d->dtype != TPA_BF16) return false;
    if (d->cache_format != TPA_CACHE_NATIVE && d->cache_format != TPA_CACHE_E4M3) return false;
    if (d->cache_format == TPA_CACHE_E4M3) {
        if (d->dtype != TPA_BF16) return false;
        for (int k = 0; k < 4; ++k)
            if (!(d->cache_scale[k] >= 0.f) || !isfinite(d->cache_scale[k])) return false;
    }
    if (!(d->rope_base > 0.0) || !isfinite(d->rope_base)) return false;
    return true;
}

Layout layout_of(const tpa_dims *d) {
    return tpa::make_layout(d->h, d->d_h, d->R_K, d->R_V, d->dtype, d->cache_format);
}

// Scale of factor k (0 A_K, 1 B_K, 2 A_V, 3 B_V): the stored value is code * scale for an E4M3 cache.
double factor_scale(const tpa_dims *d, int k) {
    if (d->cache_format != TPA_CACHE_E4M3 || d->cache_scale[k] == 0.f) return 1.0;
    return double(d->cache_scale[k]);
}

int32_t check_dims(const tpa_dims *d) {
    if (!dims_valid(d)) return TPA_ERR_ARG;
    if (!tpa::decode_supported(layout_of(d))) return TPA_ERR_UNSUPPORTED;
    return TPA_OK;
}

// Decode workspace: [partials O][partials (max, sum)][per-sequence work-group range], one partial per
// (work-group, sequence) job, at index wg + b (at most grid + batch - 1 of them).
struct DecodePlan {
    int split_blocks = 0;  // 0: the kernel's even share
    int grid = 1;
    int merge_parts = 1;
    int64_t off_o = 0;
    int64_t off_ml = 0;
    int64_t off_meta = 0;
    int64_t bytes = 0;
    bool ok = true;
};

DecodePlan plan_decode(const Layout &L, int32_t batch, int32_t max_len, int32_t split_tokens) {
    DecodePlan P;
    const int TOK = L.tok_per_block();
    const int64_t vmax = std::max<int64_t>((int64_t(max_len) + TOK - 1) / TOK, 1);  // virtual blocks per sequence
    int64_t grid, t_est;
    if (split_tokens > 0) {
        const int64_t sb = (int64_t(split_tokens) + TOK - 1) / TOK;
        grid = (int64_t(batch) * vmax + sb - 1) / sb;
        t_est = sb;
        P.split_blocks = int(std::min<int64_t>(sb, 1 << 30));
    } else {
        const int64_t target = L.HP * L.DP >= 2048 ? kWideDecodeGroups : kComputeUnits;
        grid = std::min<int64_t>(target, (int64_t(batch) * vmax + 4 * kDecodeWaves - 1) / (4 * kDecodeWaves));
        t_est = std::max<int64_t>(4 * kDecodeWaves, (int64_t(batch) * vmax + grid - 1) / grid);
    }
    if (grid < 1) grid = 1;
    const int64_t parts = grid + batch;
    // the kernel partitions the batch's virtual blocks in 32-bit arithmetic: keep every count it forms
    // (padded sequences included) below 2^31
    const int64_t vblocks = int64_t(batch) * (2 * vmax + 4 * kDecodeWaves) + t_est;
    P.ok = grid <= (int64_t(1) << 30) && parts * L.HP * L.DP <= (int64_t(1) << 40) && vblocks < (int64_t(1) << 31);
    P.grid = int(std::min<int64_t>(grid, 1 << 30));
    P.merge_parts = int(std::min<int64_t>((vmax + t_est - 1) / t_est + 1, 1 << 30));
    const int64_t o_bytes = parts * L.HP * L.DP * 4;
    P.off_o = 0;
    P.off_ml = P.off_o + (o_bytes + 255) / 256 * 256;
    P.off_meta = P.off_ml + (parts * L.HP * 2 * 4 + 255) / 256 * 256;
    P.bytes = P.off_meta + (int64_t(batch) * 8 + 255) / 256 * 256;
    return P;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// TPA_LOG set (and not "0"), checked on every call: each decode and prefill call prints its launch plan to
// stderr before launching.
bool log_on() {
    const char *e = getenv("TPA_LOG");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}
inline bool aligned16(const void *ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; }

float resolve_scale(float scale, int d_h) { return scale > 0.f ? scale : float(1.0 / sqrt(double(d_h))); }

// Device address of this device's copy of `scratch`, looked up once per device with that device current
// (the caller's current device, which must be the one its stream runs on).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_address(void *stream, void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TPA_ERR_HIP;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess) return TPA_ERR_HIP;
        if (sdev != dev) return TPA_ERR_ARG;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TPA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return TPA_OK;
}

// tpa_decode, tpa_decode_step, tpa_decode_fq and tpa_decode_noalloc: host checks, the split plan, then the
// split and merge kernels.  `step` is null for a plain decode over rotated queries.  use_scratch: the
// partials go to the static scratch array (the workspace arguments are ignored).
int32_t run_decode(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                   const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *q, float scale,
                   float *out, int32_t split_tokens, void *workspace, int64_t workspace_bytes, void *stream,
                   const tpa::StepInputs *step, int32_t r_q = 0, const void *a_q = nullptr,
                   bool use_scratch = false) {
    int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (batch < 0 || batch > 65535 || max_len < 0 || split_tokens < 0 || capacity_tokens < 0)
        return TPA_ERR_ARG;
    if (batch == 0) return TPA_OK;
    if (!cache || !seq_start || !seq_len || !q || !out) return TPA_ERR_ARG;
    if (!aligned16(cache) || !aligned16(q)) return TPA_ERR_ARG;
    if (!isfinite(scale)) return TPA_ERR_ARG;
    // a step also writes slot seq_start + seq_len, so its last possible slot must exist too
    if (int64_t(max_len) + (step ? 1 : 0) > capacity_tokens) return TPA_ERR_CAPACITY;
    const Layout L = layout_of(dims);
    const DecodePlan P = plan_decode(L, batch, max_len, split_tokens);
    if (!P.ok) return TPA_ERR_ARG;
    if (use_scratch) {
        if (P.bytes > kScratchBytes) return TPA_ERR_WORKSPACE;
        const int32_t sst = scratch_address(stream, &workspace);  // the only HIP calls before the launch
        if (sst != TPA_OK) return sst;
        workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < P.bytes) return TPA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TPA_ERR_WORKSPACE;

    tpa::DecodeParams p{};
    p.cache = cache;
    p.seq_start = seq_start;
    p.seq_len = seq_len;
    p.q = q;
    p.out = out;
    p.capacity = capacity_tokens;
    p.ws_o = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + P.off_o);
    p.ws_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + P.off_ml);
    p.ws_meta = reinterpret_cast<int2 *>(reinterpret_cast<char *>(workspace) + P.off_meta);
    p.h = dims->h;
    p.d_h = dims->d_h;
    p.RK = dims->R_K;
    p.RV = dims->R_V;
    p.batch = batch;
    p.max_len = max_len;
    p.split_blocks = P.split_blocks;
    p.grid = P.grid;
    p.merge_parts = P.merge_parts;
    p.score_mul = float(double(resolve_scale(scale, dims->d_h)) * M_LOG2E * factor_scale(dims, 0) *
                        factor_scale(dims, 1) / dims->R_K);
    p.out_mul = float(factor_scale(dims, 2) * factor_scale(dims, 3) / dims->R_V);
    if (step) {
        p.step = 1;
        p.st = *step;
        for (int k = 0; k < 4; ++k) p.st.inv_scale[k] = float(1.0 / factor_scale(dims, k));
    }
    // the fused step rotates its query, the factored query its built query row, at position seq_len[b]
    if (step || r_q > 0) p.rope = tpa::make_rope_table(dims->d_h, dims->rope_base);
    p.r_q = r_q;
    p.a_q = a_q;
    if (log_on())
        fprintf(stderr,
                "[tpa] %s: batch %d, max_len %d, heads %d->%d, d_h %d->%d, rank %d%s | %d work-groups, %s, "
                "merge work-groups of %d threads, workspace %lld B%s\n",
                step ? "decode step" : (r_q > 0 ? "factored-query decode" : "decode"), batch, max_len, dims->h, L.HP,
                dims->d_h, L.DP, L.RH, L.f8 ? ", E4M3 cache" : "", P.grid,
                P.split_blocks > 0 ? "fixed pieces of split_tokens" : "the batch's blocks shared out evenly",
                tpa::decode_merge_threads(L, p), (long long)P.bytes, use_scratch ? " (static array)" : "");
    const hipError_t e = tpa::launch_decode(L, p, as_stream(stream));
    return e == hipSuccess ? TPA_OK : TPA_ERR_HIP;
}

// tpa_prefill_chunk and tpa_prefill_chunk_fq: host checks, then the prefill kernel.  r_q > 0: q holds the
// unrotated query feature factors and a_q the query head factors.
int32_t run_prefill(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                    const int64_t *seq_start, const int32_t *ctx_len, int32_t max_ctx, int32_t chunk_len, const void *q,
                    float scale, float *out, void *stream, int32_t r_q, const void *a_q) {
    int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (batch < 0 || batch > 65535 || max_ctx < 0 || chunk_len < 0 || capacity_tokens < 0) return TPA_ERR_ARG;
    if (batch == 0 || chunk_len == 0) return TPA_OK;
    if (!cache || !seq_start || !ctx_len || !q || !out) return TPA_ERR_ARG;
    if (!aligned16(cache) || !aligned16(q) || !aligned16(out)) return TPA_ERR_ARG;
    if (!isfinite(scale)) return TPA_ERR_ARG;
    if (int64_t(max_ctx) + chunk_len > capacity_tokens) return TPA_ERR_CAPACITY;
    const Layout L = layout_of(dims);
    if (!tpa::prefill_supported(L)) return TPA_ERR_UNSUPPORTED;
    const int64_t groups = (int64_t(chunk_len) + tpa::kPrefillRows - 1) / tpa::kPrefillRows * dims->h * batch;
    if (groups * tpa::kPrefillThreads > tpa::kMaxGridItems) return TPA_ERR_ARG;
    tpa::PrefillParams p{};
    p.cache = cache;
    p.seq_start = seq_start;
    p.ctx_len = ctx_len;
    p.q = q;
    p.out = out;
    p.capacity = capacity_tokens;
    p.h = dims->h;
    p.d_h = dims->d_h;
    p.RK = dims->R_K;
    p.RV = dims->R_V;
    p.batch = batch;
    p.chunk = chunk_len;
    p.max_ctx = max_ctx;
    p.score_mul = float(double(resolve_scale(scale, dims->d_h)) * M_LOG2E * factor_scale(dims, 0) *
                        factor_scale(dims, 1) / dims->R_K);
    p.out_mul = float(factor_scale(dims, 2) * factor_scale(dims, 3) / dims->R_V);
    p.r_q = r_q;
    p.a_q = a_q;
    if (r_q > 0) p.rope = tpa::make_rope_table(dims->d_h, dims->rope_base);
    if (log_on()) {
        const int rows = tpa::prefill_rows_per_group(L, p);
        fprintf(stderr, "[tpa] %s: batch %d, chunk %d, max_ctx %d, heads %d, d_h %d->%d, rank %d%s | %lld work-groups "
                        "of %d query rows\n", r_q > 0 ? "factored-query prefill" : "prefill", batch, chunk_len, max_ctx,
                dims->h, dims->d_h, L.DP, L.RH, L.f8 ? ", E4M3 cache" : "",
                (long long)((int64_t(chunk_len) + rows - 1) / rows * dims->h * batch), rows);
    }
    const hipError_t e = tpa::launch_prefill(L, p, as_stream(stream));
    return e == hipSuccess ? TPA_OK : TPA_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t tpa_abi_version(void) { return TPA_ABI_VERSION; }

const char *tpa_status_string(int32_t status) {
    switch (status) {
        case TPA_OK: return "TPA_OK";
        case TPA_ERR_ARG: return "TPA_ERR_ARG: invalid argument";
        case TPA_ERR_UNSUPPORTED: return "TPA_ERR_UNSUPPORTED: no kernel compiled for these dims";
        case TPA_ERR_CAPACITY: return "TPA_ERR_CAPACITY: slot beyond cache capacity";
        case TPA_ERR_WORKSPACE: return "TPA_ERR_WORKSPACE: workspace missing or too small";
        case TPA_ERR_HIP: return "TPA_ERR_HIP: kernel launch failed";
    }
    return "TPA_ERR_UNKNOWN";
}

int32_t tpa_supported(const tpa_dims *dims) { return check_dims(dims) == TPA_OK ? 1 : 0; }

int32_t tpa_block_tokens(const tpa_dims *dims) {
    if (!dims_valid(dims)) return -1;
    return layout_of(dims).tok_per_block();
}

int64_t tpa_cache_bytes(const tpa_dims *dims, int64_t capacity_tokens) {
    if (!dims_valid(dims) || capacity_tokens < 0) return -1;
    const Layout L = layout_of(dims);
    const int64_t blocks = (capacity_tokens + L.tok_per_block() - 1) / L.tok_per_block();
    return blocks * L.block_elems() * L.es;
}

int32_t tpa_cache_append(const tpa_dims *dims, void *cache, int64_t capacity_tokens, int64_t n_kv,
                         const int64_t *slot, const int32_t *kv_pos, int64_t slot_hi, const void *A_K,
                         const void *B_K, const void *A_V, const void *B_V, int64_t n_q, int32_t q_rows,
                         const int32_t *q_pos, const void *q_in, void *q_out, void *stream) {
    int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (capacity_tokens < 0 || n_kv < 0 || n_q < 0) return TPA_ERR_ARG;
    if (n_kv > int64_t(0x7fffffff) || n_q > int64_t(0x7fffffff)) return TPA_ERR_ARG;
    const uintptr_t pair_bytes = 2u * uintptr_t(dims->dtype == TPA_BF16 ? 2 : 4);
    auto pair_aligned = [&](const void *ptr) { return reinterpret_cast<uintptr_t>(ptr) % pair_bytes == 0; };
    if (n_kv > 0) {
        if (!cache || !slot || !kv_pos || !A_K || !B_K || !A_V || !B_V) return TPA_ERR_ARG;
        if (!pair_aligned(B_K) || !pair_aligned(B_V) || !aligned16(cache))
            return TPA_ERR_ARG;
        if (slot_hi < 0) return TPA_ERR_ARG;
        if (slot_hi > capacity_tokens) return TPA_ERR_CAPACITY;
    }
    if (n_q > 0) {
        if (q_rows < 1 || !q_pos || !q_in || !q_out) return TPA_ERR_ARG;
        if (!pair_aligned(q_in) || !pair_aligned(q_out)) return TPA_ERR_ARG;
        if (int64_t(q_rows) * dims->d_h > int64_t(1) << 24) return TPA_ERR_ARG;
    }
    // one work-group per cache token and append_q_groups per query token, in one 1-D launch
    if ((n_kv + (n_q > 0 ? n_q * tpa::append_q_groups(q_rows, dims->d_h) : 0)) * tpa::kAppendThreads >
        tpa::kMaxGridItems)
        return TPA_ERR_ARG;
    if (n_kv == 0 && n_q == 0) return TPA_OK;
    float inv_scale[4];
    for (int k = 0; k < 4; ++k) inv_scale[k] = float(1.0 / factor_scale(dims, k));
    const hipError_t e = tpa::launch_append(layout_of(dims), dims->h, dims->d_h, dims->R_K, dims->R_V,
                                            dims->rope_base, cache, capacity_tokens, n_kv, slot, kv_pos, A_K, B_K,
                                            A_V, B_V, n_q, q_rows, q_pos, q_in, q_out, inv_scale, as_stream(stream));
    return e == hipSuccess ? TPA_OK : TPA_ERR_HIP;
}

int32_t tpa_cache_read(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int64_t n,
                       const int64_t *slot, void *A_K, void *B_K, void *A_V, void *B_V, void *stream) {
    int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (capacity_tokens < 0 || n < 0 || n * tpa::kAppendThreads > tpa::kMaxGridItems) return TPA_ERR_ARG;
    if (n == 0) return TPA_OK;
    if (!cache || !slot || !A_K || !B_K || !A_V || !B_V) return TPA_ERR_ARG;
    const hipError_t e = tpa::launch_read(layout_of(dims), dims->h, dims->d_h, dims->R_K, dims->R_V, cache,
                                          capacity_tokens, n, slot, A_K, B_K, A_V, B_V, as_stream(stream));
    return e == hipSuccess ? TPA_OK : TPA_ERR_HIP;
}

int64_t tpa_decode_workspace_bytes(const tpa_dims *dims, int32_t batch, int32_t max_len, int32_t split_tokens) {
    if (!dims_valid(dims) || batch < 0 || max_len < 0 || split_tokens < 0) return -1;
    const DecodePlan P = plan_decode(layout_of(dims), batch, max_len, split_tokens);
    return P.ok ? P.bytes : -1;
}

int32_t tpa_decode(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                   const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *q_rot,
                   float scale, float *out, int32_t split_tokens, void *workspace, int64_t workspace_bytes,
                   void *stream) {
    return run_decode(dims, cache, capacity_tokens, batch, seq_start, seq_len, max_len, q_rot, scale, out,
                      split_tokens, workspace, workspace_bytes, stream, nullptr);
}

int32_t tpa_decode_noalloc(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                           const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *q_rot,
                           float scale, float *out, int32_t split_tokens, void *stream) {
    return run_decode(dims, cache, capacity_tokens, batch, seq_start, seq_len, max_len, q_rot, scale, out,
                      split_tokens, nullptr, 0, stream, nullptr, 0, nullptr, true);
}

int32_t tpa_decode_step(const tpa_dims *dims, void *cache, int64_t capacity_tokens, int32_t batch,
                        const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *A_K,
                        const void *B_K, const void *A_V, const void *B_V, const void *q, float scale, float *out,
                        int32_t split_tokens, void *workspace, int64_t workspace_bytes, void *stream) {
    const int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (batch > 0 && (!A_K || !B_K || !A_V || !B_V)) return TPA_ERR_ARG;
    tpa::StepInputs step;
    step.A_K = A_K;
    step.B_K = B_K;
    step.A_V = A_V;
    step.B_V = B_V;
    step.cache = cache;
    step.capacity = capacity_tokens;
    return run_decode(dims, cache, capacity_tokens, batch, seq_start, seq_len, max_len, q, scale, out, split_tokens,
                      workspace, workspace_bytes, stream, &step);
}

int32_t tpa_decode_fq(const tpa_dims *dims, int32_t R_Q, const void *cache, int64_t capacity_tokens, int32_t batch,
                      const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *A_Q,
                      const void *B_Q, float scale, float *out, int32_t split_tokens, void *workspace,
                      int64_t workspace_bytes, void *stream) {
    const int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (R_Q < 1 || R_Q > 16) return TPA_ERR_ARG;
    if (batch > 0 && !A_Q) return TPA_ERR_ARG;
    return run_decode(dims, cache, capacity_tokens, batch, seq_start, seq_len, max_len, B_Q, scale, out,
                      split_tokens, workspace, workspace_bytes, stream, nullptr, R_Q, A_Q);
}

int32_t tpa_prefill_chunk(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                          const int64_t *seq_start, const int32_t *ctx_len, int32_t max_ctx, int32_t chunk_len,
                          const void *q_rot, float scale, float *out, void *stream) {
    return run_prefill(dims, cache, capacity_tokens, batch, seq_start, ctx_len, max_ctx, chunk_len, q_rot, scale,
                       out, stream, 0, nullptr);
}

int32_t tpa_prefill_chunk_fq(const tpa_dims *dims, int32_t R_Q, const void *cache, int64_t capacity_tokens,
                             int32_t batch, const int64_t *seq_start, const int32_t *ctx_len, int32_t max_ctx,
                             int32_t chunk_len, const void *A_Q, const void *B_Q, float scale, float *out,
                             void *stream) {
    const int32_t st = check_dims(dims);
    if (st != TPA_OK) return st;
    if (R_Q < 1 || R_Q > 16) return TPA_ERR_ARG;
    if (batch > 0 && chunk_len > 0 && !A_Q) return TPA_ERR_ARG;
    return run_prefill(dims, cache, capacity_tokens, batch, seq_start, ctx_len, max_ctx, chunk_len, B_Q, scale,
                       out, stream, R_Q, A_Q);
}

}  // extern "C"
