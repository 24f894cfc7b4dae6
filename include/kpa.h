/*
 * kpa.h -- C ABI of libkpa: Kronecker Product Attention (KPA) decode from a
 * cache that holds only the compact key/value factors, for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (cited by page title and section / equation):
 *   [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
 *         Structured Factorization" (arXiv 2610.12657).
 *   [TPA] "Tensor Product Attention Is All You Need" (arXiv 2501.06425) and
 *         its architecture-summary page.
 *
 * What is computed.  For every token t the cache holds the factors
 *   {A^K_r, B~^K_r} r < R_K  and  {A^V_r, B^V_r} r < R_V        ([KPA] §2.5)
 * with A_r a p1 x q1 matrix and B_r a p2 x q2 matrix (p1 = h1, p2 = h2,
 * q1 = d1, q2 = d2 in the paper's letters), so that
 *   K_t = (1/R_K) sum_r A^K_r (x) B^K_r,  V_t = (1/R_V) sum_r A^V_r (x) B^V_r
 * are h x d_h matrices, h = p1 p2, d_h = q1 q2 ([KPA] §2.2, Eqs. (3)-(4)).
 * Head i = i1 p2 + i2 and feature j = j1 q2 + j2 follow the block order of
 * the Kronecker product ([KPA] Def. 2.1).  B~^K is B^K rotated at write time
 * by the Kronecker-separable RoPE (R^(2)(pos) on each row, [KPA] Def. 2.3,
 * Thm. 2.4): consecutive feature pairs (2m, 2m+1), theta_m = base^(-2m/q2),
 * (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
 * Decode takes a dense, unrotated query q (h x d_h; the KV-only form,
 * [TPA] App. G) at position q_pos and returns, per head,
 *   out_i = sum_s softmax_s(z_{i,s}) v_{s,i},  lse_i = log sum_s exp(z_{i,s}),
 *   z_{i,s} = (R_KPA(q_pos) q_i) . (R_KPA(pos_s) k_{s,i}) / sqrt(d_h)
 * computed in factor space: q is contracted with the cached B factors and then
 * with the A factors ([KPA] Prop. 2.2 / Eq. (6)); K and V are never rebuilt.
 *
 * Conventions for every entry point.
 *   - Pointers named as device pointers are device memory owned by the
 *     caller; the library never allocates, frees or keeps them.  The library
 *     keeps no state between calls (beyond a per-device CU-count lookup).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream); no call synchronises the host.  Calls on one stream are
 *     ordered; concurrent calls writing the same cache or workspace race.
 *   - Return value: KPA_OK (0) or a negative kpa_status.  Errors the host can
 *     see return before anything is launched.  Errors only the device can see
 *     are reported through the optional `dev_status` word (bits KPA_DEV_*,
 *     OR-ed in with atomics; the caller zeroes it), and the affected element
 *     is not written.
 *   - Floating-point inputs/outputs: factor tensors in dims.dtype, queries,
 *     outputs and log-sum-exp in float32.  Arithmetic is float32 with fp32
 *     accumulation (bf16 factors are multiplied exactly in fp32 or on bf16
 *     matrix cores with fp32 accumulation).
 */
#ifndef KPA_H
#define KPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layout version of the cache buffer described under kpa_cache_layout(). */
#define KPA_LAYOUT_VERSION 1

typedef enum { KPA_F32 = 0, KPA_BF16 = 1 } kpa_dtype;

typedef enum {
    KPA_OK = 0,
    KPA_ERR_INVALID_DIMS = -1, /* non-positive split/rank, odd q2, or sizes out of range */
    KPA_ERR_NULL_PTR = -2,     /* a required pointer is NULL */
    KPA_ERR_DTYPE = -3,        /* dims.dtype is not a kpa_dtype */
    KPA_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than *_workspace_bytes() */
    KPA_ERR_UNSUPPORTED = -5,  /* valid but not supported by any kernel in this build */
    KPA_ERR_HIP = -6,          /* a HIP runtime call failed (launch, attribute query) */
    KPA_ERR_INVALID_ARG = -7   /* batch/capacity/n_q/max_ctx out of range, misaligned pointer */
} kpa_status;

/* Device-side status bits (dev_status). */
#define KPA_DEV_SLOT_OUT_OF_RANGE 1u /* append: slot < 0 or slot >= capacity; token skipped */
#define KPA_DEV_NEGATIVE_POSITION 2u /* append: position < 0; token skipped */
#define KPA_DEV_CTX_OUT_OF_RANGE 4u  /* decode: ctx_len[b] < 0 or > max_ctx; clamped */

/* The head/feature split, the ranks, the cache element type and the RoPE
 * base ([KPA] §2.2 letters: p1 = h1, p2 = h2, q1 = d1, q2 = d2). */
typedef struct {
    int32_t p1, p2; /* head split, h = p1 * p2 */
    int32_t q1, q2; /* feature split, d_h = q1 * q2; q2 even (RoPE pairs) */
    int32_t r_k;    /* key rank R_K */
    int32_t r_v;    /* value rank R_V */
    int32_t dtype;  /* kpa_dtype of the cached factors */
    float rope_base; /* theta_m = rope_base^(-2m/q2); 10000 on the pages */
} kpa_dims;

/* Limits of this build (argument checks return KPA_ERR_INVALID_DIMS above them). */
#define KPA_MAX_HEADS 128     /* h */
#define KPA_MAX_HEAD_DIM 256  /* d_h */
#define KPA_MAX_RANK 16       /* R_K, R_V */
#define KPA_MAX_HD 8192       /* h * d_h */
#define KPA_MAX_NQ 64         /* queries per sequence in kpa_decode_multiq */
/* Slots per sequence (capacity); larger values return KPA_ERR_INVALID_ARG.
 * 2^30 slots of the smallest token (8 bytes) already exceed one GPU's memory. */
#define KPA_MAX_CAPACITY (1 << 30)

/*
 * Cache buffer layout (KPA_LAYOUT_VERSION 1).  One cache holds `batch`
 * sequences of `capacity` slots each.  Slots are grouped in tiles of
 * tile_slots (32) consecutive slots; tile k of sequence b starts at byte
 * (b * n_tiles + k) * tile_bytes, n_tiles = ceil(capacity / tile_slots).
 * Inside a tile the four factor sets follow each other at comp_offset[c]
 * (c = 0 A^K, 1 B~^K, 2 A^V, 3 B^V).  Element e of a set is the row-major
 * index (r * p + row) * q + col of that token's [R][p][q] factor array.
 *   - Key sets (c = 0, 1), "feature-chunk" order: the set's elements are cut
 *     into 16-byte chunks (8 bf16 or 4 f32); chunk k of slot t sits at
 *     comp_offset[c] + k * tile_slots * 16 + t * 16.
 *   - Value sets (c = 2, 3), "token-major" order: element e of slot t sits at
 *     comp_offset[c] + (e * tile_slots + t) * elem_bytes.
 * Set sizes are rounded up to whole chunks (key sets) and the tile to 128
 * bytes, so padding is per tile, never per token.  After the last tile,
 * positions_offset holds int32 positions [batch][n_tiles * tile_slots].
 * Bytes per token without padding: (R_K + R_V)(p1 q1 + p2 q2) * elem_bytes
 * ([KPA] §2.5).
 */
typedef struct {
    int32_t version;
    int32_t tile_slots;
    int32_t elem_bytes;
    int32_t n_tiles;          /* per sequence */
    int64_t tile_bytes;
    int64_t comp_offset[4];   /* byte offsets inside a tile */
    int64_t comp_elems[4];    /* elements per token in each set */
    int64_t positions_offset; /* byte offset of the int32 positions array */
    int64_t total_bytes;      /* == kpa_cache_bytes() */
} kpa_layout_info;

/* Fill *out with the layout of a cache for (dims, batch, capacity).
 * Returns KPA_OK, KPA_ERR_NULL_PTR, KPA_ERR_DTYPE, KPA_ERR_INVALID_DIMS or
 * KPA_ERR_INVALID_ARG.  Host only; never touches the GPU. */
int kpa_cache_layout(const kpa_dims* dims, int32_t batch, int32_t capacity, kpa_layout_info* out);

/* Bytes of device memory a cache for (dims, batch, capacity) needs; 0 if the
 * arguments are invalid.  The caller allocates it (256-byte aligned; torch
 * allocations are).  Host only. */
size_t kpa_cache_bytes(const kpa_dims* dims, int32_t batch, int32_t capacity);

/*
 * kpa_cache_append -- write n_new tokens per sequence into the cache
 * ([KPA] §2.4 consequence (i), §2.5; [TPA] summary page, "RoPE Compatibility
 * and Acceleration": only B^K is rotated, once, at write time).
 *   a_k [batch][n_new][R_K][p1][q1], b_k [batch][n_new][R_K][p2][q2],
 *   a_v [batch][n_new][R_V][p1][q1], b_v [batch][n_new][R_V][p2][q2]:
 *       device, dims.dtype, unrotated factors, contiguous (the reshape of the
 *       merged factor projection, [KPA] Eq. (5) and the text after it).
 *   positions [batch][n_new] int32, device: RoPE position of each new token.
 *   slot0 [batch] int32, device: slot of the first new token of sequence b;
 *       token n goes to slot slot0[b] + n (a sum past the int32 range counts
 *       as out of range, it does not wrap).
 *   dev_status: device uint32 word or NULL (KPA_DEV_SLOT_OUT_OF_RANGE,
 *       KPA_DEV_NEGATIVE_POSITION).
 * A^K, A^V, B^V are stored bit-exactly; B~^K = R^(2)(pos) B^K is computed in
 * float64 from the stored element type and rounded once (round to nearest
 * even) to dims.dtype.  The slot's position is stored in the positions array.
 * n_new = 0 or batch = 0 is a no-op.
 */
int kpa_cache_append(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                     const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                     const int32_t* positions, const int32_t* slot0, int32_t n_new,
                     uint32_t* dev_status, void* stream);

/*
 * kpa_project_append -- project n_new tokens' hidden states to their factors
 * and write them into the cache, in one kernel ([KPA] Eq. (5) and the merged
 * form after it: every factor is a linear map of the hidden state, the ranks
 * of a factor type merged into one matrix whose product is reshaped to
 * [R][p][q]; the four merged matrices are stacked here).
 *   x [batch][n_new][d_model]: bf16, device, 16-byte aligned; the hidden
 *       states (token n of sequence b at row b * n_new + n).
 *   d_model: a positive multiple of 64.
 *   w [F][d_model]: bf16, device, 16-byte aligned, F = (R_K + R_V)(p1 q1 + p2 q2);
 *       rows W^{B^K} (R_K p2 q2 rows), W^{A^K} (R_K p1 q1), W^{A^V}
 *       (R_V p1 q1), W^{B^V} (R_V p2 q2), each block's rows in [R][p][q]
 *       row-major order.
 *   positions, slot0, dev_status, cache: as kpa_cache_append.
 * The products are accumulated in float32 on the matrix cores (bf16
 * operands).  The cache then holds what kpa_cache_append of those products
 * would store, except that B~^K = R^(2)(pos) B^K is computed in float64 from
 * the float32 products and every value is rounded once to dims.dtype (no
 * intermediate bf16 factor tensor).  Returns KPA_OK, KPA_ERR_NULL_PTR,
 * KPA_ERR_DTYPE, KPA_ERR_INVALID_DIMS, KPA_ERR_INVALID_ARG (d_model not a
 * positive multiple of 64, batch * n_new above 2^21, misaligned pointers) or
 * KPA_ERR_HIP; n_new = 0 or batch = 0 is a no-op.
 */
int kpa_project_append(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity, const void* x,
                       int32_t d_model, const void* w, const int32_t* positions, const int32_t* slot0,
                       int32_t n_new, uint32_t* dev_status, void* stream);

/* Workspace bytes kpa_decode / kpa_decode_multiq need for these arguments
 * (partial results of the split-KV decode).  num_splits as in kpa_decode.
 * Uses the current device's CU count. */
size_t kpa_decode_workspace_bytes(const kpa_dims* dims, int32_t batch, int32_t max_ctx,
                                  int32_t n_q, int32_t num_splits);

/*
 * kpa_decode -- one query per sequence, attending to slots [0, ctx_len[b])
 * ([KPA] §2.3 Prop. 2.2 / Eq. (6), §2.4 Eq. (9); [TPA] summary page,
 * FlashTPA decoding: factor-space contraction, blocked over the cache with
 * an online log-sum-exp).
 *   cache: device, written by kpa_cache_append for (dims, batch, capacity).
 *   ctx_len [batch] int32, device: attended slots per sequence.
 *   max_ctx: host upper bound of ctx_len (sizes the grid), 0 <= max_ctx <= capacity.
 *   q [batch][h][d_h] float32, device, unrotated; q_pos [batch] int32, device.
 *   out [batch][h][d_h] float32, device.  lse [batch][h] float32, device, or NULL:
 *       natural-log log-sum-exp of the scaled scores z.
 *   workspace: device, >= kpa_decode_workspace_bytes(dims, batch, max_ctx, 1, num_splits).
 *   num_splits: 0 picks the number of KV chunks per sequence from max_ctx and
 *       the CU count; > 0 forces it (clamped to [1, ceil(max_ctx / 32)]).
 *       Results agree across split counts up to rounding: float32 rounding on
 *       the vector-ALU path, the bf16 rounding of the softmax-weighted value
 *       operand (relative 2^-8 per term) on the matrix-core path.
 *   dev_status: as for kpa_cache_append (KPA_DEV_CTX_OUT_OF_RANGE), or NULL.
 * ctx_len[b] = 0 gives out = 0 and lse = -inf.
 */
int kpa_decode(const kpa_dims* dims, const void* cache, int32_t batch, int32_t capacity,
               const int32_t* ctx_len, int32_t max_ctx, const float* q, const int32_t* q_pos,
               float* out, float* lse, void* workspace, size_t workspace_bytes,
               int32_t num_splits, uint32_t* dev_status, void* stream);

/*
 * kpa_decode_multiq -- n_q queries per sequence (chunked or speculative
 * decode).  Same arguments as kpa_decode, with
 *   q [batch][n_q][h][d_h], q_pos [batch][n_q], out [batch][n_q][h][d_h],
 *   lse [batch][n_q][h] (or NULL).
 *   causal != 0: query n sees slots s < ctx_len[b] - n_q + n + 1 (the n_q
 *   newest slots hold the queries' own tokens, appended beforehand);
 *   causal == 0: every query sees slots s < ctx_len[b].
 * The pages do not describe a multi-query kernel; the causal rule is the
 * ordinary decoder-attention mask.
 */
int kpa_decode_multiq(const kpa_dims* dims, const void* cache, int32_t batch, int32_t capacity,
                      const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                      const float* q, const int32_t* q_pos, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                      uint32_t* dev_status, void* stream);

/*
 * kpa_decode_factored -- decode with a factored query: the query of each
 * (sequence, query) row has the keys' Kronecker form,
 *   Q = (1/R_Q) sum_r A^Q_r (x) B^Q_r,  A^Q_r: p1 x q1,  B^Q_r: p2 x q2
 * ([KPA] Eq. (5)-(6), Prop. 2.2: scores then follow from head-level
 * A^Q . A^K and feature-level B^Q . B~^K products; [TPA] summary page,
 * factored queries).  Arguments as kpa_decode_multiq, with
 *   r_q: 1 <= R_Q <= KPA_MAX_RANK;
 *   a_q [batch][n_q][r_q][p1][q1], b_q [batch][n_q][r_q][p2][q2]: float32,
 *       device, 16-byte aligned, unrotated (RoPE at q_pos is applied to B^Q,
 *       as to B^K);
 *   n_q >= 1 queries per sequence, causal as for kpa_decode_multiq (ignored
 *       for n_q = 1).
 * The same kernels as the dense decode run; each workgroup expands the
 * query elements it needs from the factors in its prologue.  The workspace
 * is sized by kpa_decode_workspace_bytes(dims, batch, max_ctx, n_q, num_splits).
 * Returns as kpa_decode; KPA_ERR_INVALID_DIMS for r_q out of range.
 */
int kpa_decode_factored(const kpa_dims* dims, int32_t r_q, const void* cache, int32_t batch, int32_t capacity,
                        const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                        const float* a_q, const float* b_q, const int32_t* q_pos, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, int32_t num_splits,
                        uint32_t* dev_status, void* stream);

/*
 * kpa_append_decode -- one decode step: kpa_cache_append of n_new tokens per
 * sequence, then kpa_decode_multiq over the updated cache (the pages' decode
 * step writes the new token's factors to the cache and attends over it:
 * [KPA] §2.5; [TPA] summary page, "RoPE Compatibility and Acceleration").
 * Arguments: those of kpa_cache_append (cache writable, a_k .. slot0, n_new
 * >= 0; n_new = 0 needs none of a_k .. slot0) and of kpa_decode_multiq
 * (n_q = 1 is the single-query decode).  Results, cache bytes and dev_status
 * bits equal those of the two calls made in that order on the same stream.
 * With one query per sequence on the matrix-core kernels the append is fused
 * into the decode kernel (one launch fewer): each new token is written by
 * the workgroup whose KV chunk holds its slot, before it reads it; other
 * paths launch the append kernel first.  Returns as kpa_decode_multiq; KPA_ERR_INVALID_ARG for n_new < 0,
 * KPA_ERR_NULL_PTR for a missing append input when n_new > 0 and batch > 0.
 */
int kpa_append_decode(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                      const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                      const int32_t* positions, const int32_t* slot0, int32_t n_new,
                      const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                      const float* q, const int32_t* q_pos, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                      uint32_t* dev_status, void* stream);

/* Device scratch of kpa_append_decode_noalloc, per GPU (32 MiB). */
#define KPA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * kpa_append_decode_noalloc -- kpa_append_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without
 * workspace / workspace_bytes; the split-KV partials live in a static
 * device array of KPA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends (its address is looked up once per
 * device, on that device's first call).  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  Results and cache
 * bytes equal kpa_append_decode's with the same num_splits.  Returns as
 * kpa_append_decode, and KPA_ERR_WORKSPACE (nothing launched) when the
 * partials of this call would exceed KPA_NOALLOC_SCRATCH_BYTES
 * (kpa_decode_workspace_bytes() tells the size).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
int kpa_append_decode_noalloc(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                              const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                              const int32_t* positions, const int32_t* slot0, int32_t n_new,
                              const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                              const float* q, const int32_t* q_pos, float* out, float* lse,
                              int32_t num_splits, uint32_t* dev_status, void* stream);

/*
 * kpa_time_next_decode_kernel -- measurement hook.  start_event and
 * stop_event are hipEvent_t handles created by the caller with timing
 * enabled (both non-NULL), or both NULL to cancel a pending request.  The
 * next decode call (kpa_decode, kpa_decode_multiq, kpa_decode_factored,
 * kpa_append_decode), kpa_project_append or kpa_stream_xor call made on the
 * same host thread launches its main kernel (the split-KV decode kernel; the
 * projection kernel; the streaming read) with hipExtLaunchKernel, so that the runtime stamps start_event
 * and stop_event with that kernel's own start and end on its stream (the
 * log-sum-exp merge is not included).  The request is then dropped, also
 * when that call fails its checks.  The stamped events still cost the stream
 * a few microseconds between dispatches: time a sample of calls, not every
 * one.  The events stay owned by the caller and must outlive that call.
 * Returns KPA_OK, or KPA_ERR_NULL_PTR if exactly one handle is NULL.
 */
int kpa_time_next_decode_kernel(void* start_event, void* stop_event);

/*
 * kpa_stream_xor -- measurement aid, not part of the method: the rate of a
 * plain streaming read, against which the decode kernels' HBM rate is set
 * (run it over the same buffer a decode reads, e.g. the cache).  Reads the
 * `bytes` bytes at `buf` once, with 16-byte nontemporal loads (the decode
 * kernels' load form).  n_blocks workgroups each take one contiguous share:
 * with n16 = bytes / 16 and C = ceil(n16 / n_blocks), workgroup w reads the
 * 16-byte words [w C, min((w + 1) C, n16)) and writes to partial[w] the XOR
 * of their 32-bit words (0 for an empty share), so the XOR of partial[] is
 * the XOR of every 32-bit word of the buffer.
 *   buf      device, 16-byte aligned, `bytes` readable; bytes a positive
 *            multiple of 16, at most 2^40
 *   partial  device uint32_t[n_blocks], written
 *   n_blocks 1 .. 65535 (the chip holds 8 such workgroups per CU at once;
 *            3 per CU is the decode kernels' usual grid)
 * Consumes a pending kpa_time_next_decode_kernel request.  Returns KPA_OK,
 * KPA_ERR_NULL_PTR, KPA_ERR_INVALID_ARG (sizes, alignment), KPA_ERR_HIP.
 */
int kpa_stream_xor(const void* buf, size_t bytes, uint32_t* partial, int32_t n_blocks, void* stream);

/* Static description of a kpa_status code. */
const char* kpa_status_string(int status);

/*
 * kpa_decode_path -- name of the kernel path the decode entry points run for
 * these dims and n_q, or "" for invalid arguments.  Host only.
 *   "mfma_rebuild": several queries per sequence on the bf16 matrix cores with
 *       K and V rebuilt per tile from their factors (Eqs. (3)-(4): per token
 *       and head a sum of R outer products, formed by matrix instructions)
 *       and plain attention over the rebuilt rows (the rebuilt rows, the
 *       rotated query and the softmax weights each rounded once to bf16;
 *       float32 sums).  Taken for bf16 caches with R_K <= 4, R_V <= 4 and
 *       either n_q >= 8, q1 = 16, q2 = 8, p2 = 2, 4, 6 or 8, any p1, or
 *       n_q >= 12, q1 = 8, q2 = 16, p1 = 8, any p2 (the factors' roles
 *       swapped); every rebuilt row then serves 8-16 queries.
 *   "mfma_bf16": the bf16 matrix cores.  Taken by every other bf16 cache where
 *       one factor -- call it F -- has a feature dimension of 8, 16, 32 or 64
 *       (contracted on the matrix cores) and
 *         - the other factor's feature dimension q_G is 1, 2, 4, 8, 16 or 32;
 *         - R_K <= 4 and R_V <= 4;
 *         - its rows M = p_G q_G (p_G = the other factor's head count) are
 *           at most 128 when F's feature dimension is 8 or 16, at most 64
 *           when it is 32 or 64 (32 for n_q > 1), and a multiple of 4
 *           unless R_K = 1;
 *         - F's head count p_F is at most 8 for one query (4 when the
 *           shape's rows exceed 64 or a rank exceeds 2, or F is 32 or 64
 *           wide) and at most 4 for n_q > 1; the other factor's head count
 *           p_G is at most 64 for one query and 32 for n_q > 1;
 *         - the kernel's LDS for the shape (two staged tiles of the G
 *           factors plus per-wave score rows, growing with the rows and
 *           ranks) fits the 160 KB of a compute unit;
 *       plus the exact shapes the library is tuned for (the workload
 *       configurations, the KPA page's head splits and FlashTPA's shapes).
 *       When both factors qualify, the one giving an even spread of waves
 *       over a CU's four SIMDs, then fewer padded rows, is chosen.
 *   "valu": the vector ALUs: float32 caches, and bf16 shapes outside the
 *       families above (e.g. no feature dimension of 8/16/32/64, a rank above
 *       4, a non-power-of-two q_G).  Every shape within the kpa_dims limits
 *       runs on one of these paths; results agree within the stated
 *       tolerances.
 */
const char* kpa_decode_path(const kpa_dims* dims, int32_t n_q);

#ifdef __cplusplus
}
#endif

#endif /* KPA_H */
