/*
 * tpa.h -- C ABI of libtpa: attention evaluated directly over a factorized
 * KV cache in Tensor Product Attention (TPA) form, on AMD Instinct MI355X
 * (gfx950).
 *
 * The method ("Tensor Product Attention Is All You Need", paper notes page):
 *   - Key design, tensor product decomposition: each token's key is
 *     K_t = (1/R_K) A_K(x_t)^T B_K(x_t) with a head factor A_K in R^{R_K x h}
 *     and a feature factor B_K in R^{R_K x d_h}; V likewise with R_V.  The
 *     cache keeps only A_K, B_K, A_V, B_V: (R_K + R_V)(h + d_h) elements per
 *     token instead of 2 h d_h.
 *   - Key design, RoPE compatibility (Theorem 3.1): rotating only the B
 *     factors by position keeps RoPE's relative-position property,
 *     Q~_t K~_s^T = Q_t T_{t-s} K_s^T.
 *   - Key design, FlashTPA: attention is computed from the factors without
 *     ever building the full K or V.
 * Readings where the pages are silent: RoPE uses RoFormer pairs (2j, 2j+1)
 * with theta_j = rope_base^(-2j/d_h) over all d_h features; the softmax
 * scale defaults to 1/sqrt(d_h) and 1/R_K, 1/R_V are applied inside.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  Element arrays hold
 *     `dims->dtype` elements (fp32 or bf16); outputs are fp32.
 *   - The caller owns every buffer (allocate with hipMalloc or a framework
 *     allocator).  The library allocates nothing, never synchronizes, and
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *     stream).  Completion is asynchronous.  Its only mutable global state is
 *     the per-device address of the static partials array of
 *     tpa_decode_noalloc.
 *   - The cache, q_rot and prefill's out must be 16-byte aligned (wide vector
 *     loads and stores); hipMalloc and framework allocators give 256 bytes.
 *   - Every call returns a tpa_status.  All argument checks run on the host
 *     before any HIP call; a rejected call launches nothing.  TPA_ERR_HIP
 *     reports a failed launch (hipGetLastError).  Values held in device
 *     memory (slots, starts, lengths) cannot be checked on the host; the
 *     kernels check them against capacity_tokens: an append skips a slot
 *     outside the cache, and a decode or prefill sequence whose slots are
 *     not all inside it (or whose start is not a block boundary) gets NaN
 *     output while no slot outside the cache is read or written.
 *
 * Cache layout (opaque; written by tpa_cache_append, read back by
 * tpa_cache_read).  Tokens are grouped into blocks of tpa_block_tokens()
 * consecutive slots; inside a block the factors are stored in the order the
 * decode kernel's matrix-core operands consume them, so every load is a
 * contiguous 1 KiB wave read.  A sequence occupies consecutive slots
 * starting at a block boundary; slot order is position order.
 */
#ifndef TPA_H
#define TPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPA_ABI_VERSION 3

typedef enum tpa_status {
    TPA_OK = 0,
    TPA_ERR_ARG = 1,         /* null pointer, bad dimension or count, misaligned size, or a call whose
                                launch would count more than 2^32 - 1 work-items (append and read: 128
                                per cache token; prefill: 512 per 256 query rows of one head) */
    TPA_ERR_UNSUPPORTED = 2, /* valid shape with no compiled kernel (see tpa_supported) */
    TPA_ERR_CAPACITY = 3,    /* a slot at or beyond the cache capacity */
    TPA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than tpa_decode_workspace_bytes */
    TPA_ERR_HIP = 5          /* a kernel launch failed */
} tpa_status;

typedef enum tpa_dtype { TPA_F32 = 0, TPA_BF16 = 1 } tpa_dtype;

/* How the cache stores factor elements.
 *   TPA_CACHE_NATIVE  in dims->dtype (fp32 or bf16).
 *   TPA_CACHE_E4M3    one byte per element: the OCP 8-bit floating-point E4M3
 *                     code of value / scale (1 sign, 4 exponent bits with bias 7,
 *                     3 mantissa bits; largest finite magnitude 448, no
 *                     infinities), rounded to nearest even and saturating at 448;
 *                     the stored value is code * scale, with one scale per factor
 *                     tensor (dims->cache_scale).  Requires dtype TPA_BF16 (inputs
 *                     and queries stay bf16).  This is the low-bit factor storage
 *                     the TPA notes page lists as unexplored (Limitations): it
 *                     halves the bytes per cached token again, with the rounding
 *                     error of a 3-bit mantissa on every factor element. */
typedef enum tpa_cache_format { TPA_CACHE_NATIVE = 0, TPA_CACHE_E4M3 = 1 } tpa_cache_format;

/* Problem statement of one attention layer (TPA notes page, tensor product
 * decomposition and RoPE compatibility):
 *   h             number of heads, 1..64
 *   d_h           head dimension, even, 2..256
 *   R_K, R_V      factor ranks of K and V, 1..4
 *   dtype         element type of factors and queries (and of the cache, when native)
 *   cache_format  a tpa_cache_format
 *   rope_base     RoPE base (theta_j = rope_base^(-2j/d_h)), > 0
 *   cache_scale   TPA_CACHE_E4M3 only: scales of A_K, B_K, A_V, B_V (finite, >= 0;
 *                 0 means 1).  Ignored for a native cache. */
typedef struct tpa_dims {
    int32_t h;
    int32_t d_h;
    int32_t R_K;
    int32_t R_V;
    int32_t dtype;
    int32_t cache_format;
    double rope_base;
    float cache_scale[4];
} tpa_dims;

int32_t tpa_abi_version(void);

/* Human-readable name of a status code.  Never NULL. */
const char *tpa_status_string(int32_t status);

/* 1 if kernels exist for these dims, 0 if not (also 0 for invalid dims). */
int32_t tpa_supported(const tpa_dims *dims);

/* Tokens per cache block: sequences must start at a multiple of it.  <= 0 on bad dims. */
int32_t tpa_block_tokens(const tpa_dims *dims);

/* Bytes of device memory a cache of capacity_tokens slots needs (capacity is
 * rounded up to whole blocks).  For h a multiple of 16 and d_h a multiple of
 * 32 (bf16) or 16 (fp32), and R_K = R_V in {1, 2, 4}, this is exactly
 * capacity * (R_K + R_V)(h + d_h) * sizeof(element): the factor-only size of
 * the tensor product decomposition paragraph.  Other shapes are padded.
 * -1 on bad dims or a negative capacity. */
int64_t tpa_cache_bytes(const tpa_dims *dims, int64_t capacity_tokens);

/* Write factors of n_kv tokens into the cache and, optionally, rotate query rows.
 * (TPA notes page: the cache holds only A_K, B_K, A_V, B_V; RoPE compatibility:
 * B_K is rotated by the token's position, and so are query rows.)
 *   cache, capacity_tokens   the cache (tpa_cache_bytes(dims, capacity_tokens) bytes)
 *   slot[n_kv]     int64, cache slot of each token; a slot < 0 or >= capacity is skipped
 *   kv_pos[n_kv]   int32, position of each token (>= 0)
 *   slot_hi        [host] an upper bound on max(slot)+1; must be <= capacity_tokens
 *   A_K [n_kv][R_K][h], B_K [n_kv][R_K][d_h], A_V [n_kv][R_V][h], B_V [n_kv][R_V][d_h]
 *                  unrotated factors, contiguous; B_K is rotated on the way in
 *   n_q            number of query tokens to rotate (0: none; q pointers may then be NULL)
 *   q_rows         rows per query token: h for a full query, or R_Q for a B_Q factor
 *   q_pos[n_q]     int32 positions
 *   q_in, q_out    [n_q][q_rows][d_h]; q_out = RoPE(q_in); q_out may equal q_in
 *   B_K, B_V, q_in and q_out must be aligned to two elements (rotary pairs are
 *   moved as one word) and the cache to 16 bytes; TPA_ERR_ARG otherwise.
 * Angles are formed and reduced mod 2 pi in fp64; cos, sin and the rotation are
 * fp32 for bf16 (fp64 for fp32), rounded once to dtype.  With TPA_CACHE_E4M3
 * every factor element is stored as the code of value / scale (B_K: its fp32
 * rotation divided by the scale); queries stay dtype. */
int32_t tpa_cache_append(const tpa_dims *dims, void *cache, int64_t capacity_tokens, int64_t n_kv,
                         const int64_t *slot, const int32_t *kv_pos, int64_t slot_hi, const void *A_K,
                         const void *B_K, const void *A_V, const void *B_V, int64_t n_q, int32_t q_rows,
                         const int32_t *q_pos, const void *q_in, void *q_out, void *stream);

/* Read n tokens back out of the cache in natural layout (B_K as stored, i.e.
 * rotated).  Same array shapes as tpa_cache_append, in the stored element type:
 * dims->dtype for a native cache, one uint8 E4M3 code per element for
 * TPA_CACHE_E4M3 (value = code * scale); slots out of range read as zeros.
 * For tests and cache export. */
int32_t tpa_cache_read(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int64_t n,
                       const int64_t *slot, void *A_K, void *B_K, void *A_V, void *B_V, void *stream);

/* Workspace bytes tpa_decode needs for (batch, max_len, split_tokens).  -1 on bad arguments. */
int64_t tpa_decode_workspace_bytes(const tpa_dims *dims, int32_t batch, int32_t max_len, int32_t split_tokens);

/* Split-sequence decode: one query row per sequence attends to all of its
 * cached tokens, computed from the factors (TPA notes page, FlashTPA: no full
 * K/V is built).  The batch's cache blocks are shared out evenly over the
 * work-groups whatever the lengths (a work-group may cover the end of one
 * sequence and the start of the next); each piece leaves a partial, and a
 * second kernel merges the pieces of each sequence.  Per sequence b and head i:
 *     out[b][i] = sum_s softmax_s(scale * q~_b,i . K~_s[i,:]) V_s[i,:]
 * over s = 0 .. seq_len[b]-1, with K~_s, V_s from the cached factors.
 *   seq_start[batch]  int64 first slot of each sequence; must be a multiple of
 *                     tpa_block_tokens()
 *   seq_len[batch]    int32 cached tokens of each sequence (0 gives a zero output;
 *                     values above max_len are clamped to max_len)
 *                     A sequence with a misaligned start, or with
 *                     seq_start + seq_len > capacity_tokens, gets NaN output and
 *                     none of its slots is read (checked on the device).
 *   max_len           [host] >= every seq_len; sizes the launch
 *   q_rot [batch][h][d_h]  queries already rotated to their positions (tpa_cache_append)
 *   scale             softmax scale; <= 0 selects 1/sqrt(d_h)
 *   out [batch][h][d_h]    fp32
 *   split_tokens      cached tokens per work-group (rounded up to whole blocks); 0 lets the
 *                     library share the batch's tokens evenly over one round of work-groups
 *   workspace         >= tpa_decode_workspace_bytes(dims, batch, max_len, split_tokens)
 *                     bytes of device memory, 256-byte aligned; holds the pieces' partials
 *                     (running max, sum, unnormalized output) and each sequence's range of
 *                     pieces between the split kernel and the merge kernel.  One workspace
 *                     serves one call at a time: calls that overlap on it race.
 * max_len <= capacity_tokens, else TPA_ERR_CAPACITY. */
int32_t tpa_decode(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                   const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *q_rot,
                   float scale, float *out, int32_t split_tokens, void *workspace, int64_t workspace_bytes,
                   void *stream);

/* tpa_decode for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same split and merge kernels, with the pieces' partials in a
 * static device array of the library instead of a caller workspace.  The call allocates nothing and calls
 * no allocating routine.
 *   - The array holds TPA_DECODE_NOALLOC_MAX_BYTES; a call whose tpa_decode_workspace_bytes(dims, batch,
 *     max_len, split_tokens) exceeds it is rejected with TPA_ERR_WORKSPACE before any launch.
 *   - Each GPU holds its own copy, from the library's first use on that device until the process ends; its
 *     address is looked up on the first call on a device.  The caller's current device must be the device
 *     `stream` runs on (TPA_ERR_ARG otherwise; TPA_ERR_HIP if the lookup fails).
 *   - Every call on one GPU shares that GPU's copy: calls that overlap on one GPU (other streams, other
 *     threads) race and give wrong results.  Nothing in it needs clearing: each call writes every partial
 *     it reads.
 * Arguments, results and the other error behaviour are those of tpa_decode. */
#define TPA_DECODE_NOALLOC_MAX_BYTES (16ll << 20)
int32_t tpa_decode_noalloc(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                           const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *q_rot,
                           float scale, float *out, int32_t split_tokens, void *stream);

/* Fused single decode step (one new token per sequence): for each sequence b with N = seq_len[b] cached
 * tokens, write the new token's factors into slot seq_start[b] + N (B_K rotated at position N, exactly as
 * tpa_cache_append writes it), rotate the query at position N, and attend over the N cached tokens and
 * the new one (the one-query decode of the TPA notes page, FlashTPA; RoPE compatibility, Theorem 3.1):
 *     out[b][i] = sum_{s <= N} softmax_s(scale * q~_b,i . K~_s[i,:]) V_s[i,:]
 * Two kernel launches (split, merge) and no separate append: every work-group rotates the query in
 * registers, the work-group holding the sequence's first piece folds in the new token's own score and value
 * (query and token share a position, so RoPE cancels in that score) and the one holding its last piece
 * writes the token's record.  Over a
 * TPA_CACHE_E4M3 cache the token enters as its stored values (codes decoded back, B_K rotated before its
 * rounding), exactly as tpa_cache_append followed by tpa_decode would see it.
 *   A_K [batch][R_K][h], B_K [batch][R_K][d_h], A_V [batch][R_V][h], B_V [batch][R_V][d_h]
 *                     the new token's factors, unrotated
 *   q [batch][h][d_h]  the step's query, unrotated (16-byte aligned)
 *   seq_len[batch]     cached tokens before the step; not modified (the caller advances it)
 *   max_len [host]     >= every seq_len; max_len + 1 <= capacity_tokens (TPA_ERR_CAPACITY otherwise)
 * Other arguments, the workspace (tpa_decode_workspace_bytes(dims, batch, max_len, split_tokens)) and the
 * error behaviour are those of tpa_decode, except that the new token's slot must also be inside the cache
 * (seq_start + seq_len + 1 <= capacity_tokens, else NaN output and nothing written). */
int32_t tpa_decode_step(const tpa_dims *dims, void *cache, int64_t capacity_tokens, int32_t batch,
                        const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *A_K,
                        const void *B_K, const void *A_V, const void *B_V, const void *q, float scale, float *out,
                        int32_t split_tokens, void *workspace, int64_t workspace_bytes, void *stream);

/* Factored-query decode (full TPA: the query is factorized like K and V; TPA notes page, tensor product
 * decomposition, and its ablation's Q+K+V-factorized variant).  Per sequence b and head i the query row is
 *     q~_b,i = RoPE_N((1/R_Q) sum_r A_Q[b][r][i] B_Q[b][r][:]),   N = seq_len[b]
 * built on chip and never in device memory: fp32 sums, the rotation at the query's position N with the
 * append's arithmetic (RoPE is linear, so rotating the combined row is rotating the factor rows: RoPE
 * compatibility), one rounding to dtype.  Then the same attention as tpa_decode over the N cached tokens.
 *   R_Q [host]             query rank, 1..16 (TPA_ERR_ARG otherwise)
 *   A_Q [batch][R_Q][h]    query head factor
 *   B_Q [batch][R_Q][d_h]  query feature factor, unrotated (16-byte aligned)
 * Other arguments, the workspace (tpa_decode_workspace_bytes) and the error behaviour are tpa_decode's. */
int32_t tpa_decode_fq(const tpa_dims *dims, int32_t R_Q, const void *cache, int64_t capacity_tokens, int32_t batch,
                      const int64_t *seq_start, const int32_t *seq_len, int32_t max_len, const void *A_Q,
                      const void *B_Q, float scale, float *out, int32_t split_tokens, void *workspace,
                      int64_t workspace_bytes, void *stream);

/* Causal chunked prefill: chunk_len query rows per sequence attend to the
 * sequence's cached context and to the chunk's own tokens up to and including
 * their own (the chunk's factors must already be in the cache, appended at
 * slots seq_start[b] + ctx_len[b] + j).  Row j of sequence b sees slots
 * seq_start[b] + 0 .. seq_start[b] + ctx_len[b] + j:
 *     out[b][j][i] = sum_{s <= ctx_len[b] + j} softmax_s(scale * q~_b,j,i . K~_s[i,:]) V_s[i,:]
 * The pages state no prefill algorithm: they give the factor form of K and V
 * (tensor product decomposition), RoPE on the B factors (RoPE compatibility)
 * and the principle that attention is computed from the factors without
 * materializing K and V (FlashTPA).  This entry point applies them to a chunk
 * of query rows under the textbook causal mask: K~ and V for one head are
 * rebuilt from the factors on chip, never in device memory.
 *   ctx_len[batch]   int32 cached tokens before the chunk (<= max_ctx)
 *   max_ctx          [host] >= every ctx_len; max_ctx + chunk_len <= capacity_tokens
 *                    (TPA_ERR_CAPACITY otherwise)
 *   chunk_len        [host] rows per sequence
 *   q_rot [batch][chunk_len][h][d_h]  rotated query rows (row j at position ctx_len[b] + j)
 *   out   [batch][chunk_len][h][d_h]  fp32
 * A sequence with a misaligned start, or with seq_start + ctx_len + chunk_len >
 * capacity_tokens, gets NaN rows and none of its slots is read.
 * Currently bf16 only (TPA_ERR_UNSUPPORTED for fp32). */
int32_t tpa_prefill_chunk(const tpa_dims *dims, const void *cache, int64_t capacity_tokens, int32_t batch,
                          const int64_t *seq_start, const int32_t *ctx_len, int32_t max_ctx, int32_t chunk_len,
                          const void *q_rot, float scale, float *out, void *stream);

/* Causal chunked prefill with factored query rows (full TPA, TPA notes page, tensor product decomposition
 * applied to Q; the factored form of tpa_decode_fq): row j of sequence b has
 *     q~_b,j,i = RoPE_{ctx_len[b]+j}((1/R_Q) sum_r A_Q[b][j][r][i] B_Q[b][j][r][:])
 * built on chip (fp32 sums and rotation, one rounding to bf16), then the attention of tpa_prefill_chunk.
 *   R_Q [host]                        query rank, 1..16
 *   A_Q [batch][chunk_len][R_Q][h]    query head factors
 *   B_Q [batch][chunk_len][R_Q][d_h]  query feature factors, unrotated (16-byte aligned)
 * Other arguments and the error behaviour are tpa_prefill_chunk's. */
int32_t tpa_prefill_chunk_fq(const tpa_dims *dims, int32_t R_Q, const void *cache, int64_t capacity_tokens,
                             int32_t batch, const int64_t *seq_start, const int32_t *ctx_len, int32_t max_ctx,
                             int32_t chunk_len, const void *A_Q, const void *B_Q, float scale, float *out,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TPA_H */
