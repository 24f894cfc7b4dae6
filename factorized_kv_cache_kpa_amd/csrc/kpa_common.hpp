// Shared host/device definitions of libkpa: cache layout arithmetic, the
// launch-parameter structs and small device helpers.
//
// [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
//       Structured Factorization" (arXiv 2610.12657).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kpa.h"

namespace kpa {

constexpr int kTileSlots = 32;   // slots per cache tile
constexpr int kChunkBytes = 16;  // key sets are cut into 16-byte chunks
constexpr int kTileAlign = 128;  // tiles are padded to 128 bytes

// Cache layout (the KPA_LAYOUT_VERSION 1 description in kpa.h).
struct Layout {
    int32_t elem_bytes;
    int32_t n_tiles;       // per sequence
    int64_t tile_bytes;
    int64_t off[4];        // A^K, B~^K, A^V, B^V inside a tile
    int32_t elems[4];      // elements per token of each set
    int64_t positions_off; // start of the int32 positions array
    int64_t total_bytes;
};

inline __host__ __device__ int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Host-side construction; assumes dims already validated.
inline Layout make_layout(const kpa_dims& d, int32_t batch, int32_t capacity) {
    Layout L{};
    L.elem_bytes = d.dtype == KPA_F32 ? 4 : 2;
    L.n_tiles = (int32_t)(((int64_t)capacity + kTileSlots - 1) / kTileSlots);
    L.elems[0] = d.r_k * d.p1 * d.q1;
    L.elems[1] = d.r_k * d.p2 * d.q2;
    L.elems[2] = d.r_v * d.p1 * d.q1;
    L.elems[3] = d.r_v * d.p2 * d.q2;
    int64_t off = 0;
    for (int c = 0; c < 4; ++c) {
        L.off[c] = off;
        int64_t bytes;
        if (c < 2)  // feature-chunk: whole 16-byte chunks per slot
            bytes = round_up((int64_t)L.elems[c] * L.elem_bytes, kChunkBytes) * kTileSlots;
        else        // token-major
            bytes = (int64_t)L.elems[c] * L.elem_bytes * kTileSlots;
        off += bytes;
    }
    L.tile_bytes = round_up(off, kTileAlign);
    L.positions_off = (int64_t)batch * L.n_tiles * L.tile_bytes;
    L.total_bytes = L.positions_off + (int64_t)batch * L.n_tiles * kTileSlots * 4;
    return L;
}

// Byte offset of element e of set c for slot t inside a tile.
inline __host__ __device__ int64_t elem_offset(const Layout& L, int c, int64_t e, int t) {
    if (c < 2) {
        const int per_chunk = kChunkBytes / L.elem_bytes;
        return L.off[c] + (e / per_chunk) * (kTileSlots * kChunkBytes) + (int64_t)t * kChunkBytes +
               (e % per_chunk) * L.elem_bytes;
    }
    return L.off[c] + (e * kTileSlots + t) * L.elem_bytes;
}

// ---------------------------------------------------------------------------
// Element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float64 -> bfloat16, one rounding to nearest even.  Round to float with
// round-to-odd (truncate, then force the last bit when inexact), then round
// that float to bf16: float keeps 16 more bits than bf16, so the second
// rounding cannot double-round.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    float t = __double2float_rz(x);
    uint32_t u = __float_as_uint(t);
    if ((double)t != x) u |= 1u;
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);  // inf / nan
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Launch parameters
// ---------------------------------------------------------------------------
// New tokens for the cache: token n of sequence b goes to slot slot0[b] + n
// at position positions[b * n_new + n]; factor tensors [batch][n_new][...].
struct AppendInputs {
    const void *a_k, *b_k, *a_v, *b_v;
    const int32_t* positions;
    const int32_t* slot0;
    int32_t n_new;
};

// slot0 + n (n >= 0) for a slot0 read from device memory: a sum past the
// int32 range saturates to INT32_MAX, which is past every capacity, so the
// token is reported out of range instead of wrapping to a valid slot.
__device__ __forceinline__ int slot_add(int slot0, int n) {
    const int64_t s = (int64_t)slot0 + n;
    return s > INT32_MAX ? INT32_MAX : (int)s;
}

struct AppendParams {
    kpa_dims d;
    Layout L;
    uint8_t* cache;
    int32_t batch, capacity;
    AppendInputs in;
    uint32_t* dev_status;
};

// kpa_project_append: hidden states x [n_tok][d_model] and the stacked
// weight w [n_feat][d_model] (rows B^K, A^K, A^V, B^V), bf16.
struct ProjectParams {
    kpa_dims d;
    Layout L;
    uint8_t* cache;
    int32_t capacity, n_new, n_tok, n_feat, d_model;
    const uint16_t* x;
    const uint16_t* w;
    const int32_t* positions;
    const int32_t* slot0;
    uint32_t* dev_status;
};

struct DecodeParams {
    kpa_dims d;
    Layout L;
    const uint8_t* cache;
    int32_t batch, capacity, max_ctx;
    int32_t n_q, causal;
    const int32_t* ctx_len;
    const float* q;       // dense query [batch][n_q][h][d_h], or null with a_q/b_q
    const float* a_q;     // factored query: [batch][n_q][r_q][p1][q1]
    const float* b_q;     //                 [batch][n_q][r_q][p2][q2]
    int32_t r_q;
    const int32_t* q_pos;
    float* out;
    float* lse;
    uint32_t* dev_status;
    // split-KV
    int32_t n_split;      // chunks per (sequence, query)
    int32_t chunk_tiles;  // tiles per chunk
    float* part_o;        // [batch][n_q][n_split][h][d_h]  (unnormalised sum p v)
    float* part_ml;       // [batch][n_q][n_split][h][2]   (running max in log2 units, sum p)
    int32_t n_group;      // merge groups per (row, head); > 1 adds a second level
    float* part2_o;       // [batch][n_q][n_group][h][d_h]
    float* part2_ml;      // [batch][n_q][n_group][h][2]
    uint32_t* merge_count; // [batch][n_q][h] arrival counters of the second level
    float q_scale;        // log2(e) / (R_K sqrt(d_h))
    float v_scale;        // 1 / R_V
    // fused append (kpa_append_decode): app.n_new > 0 has the workgroups write
    // the new tokens of their own chunk into cache_w before reading them
    AppendInputs app;
    uint8_t* cache_w;
    // matrix-core kernels of a generic family: 1 = B is the factor contracted
    // on the matrix cores, 0 = A (set by the launcher)
    int32_t f_is_b;
};

// Element (i, j) of the unrotated query of row (b, n): the dense query's, or,
// for a factored query, (1/R_Q) sum_r A^Q_r[i1, j1] B^Q_r[i2, j2] with
// i = i1 p2 + i2, j = j1 q2 + j2 ([KPA] Def. 2.1, Eq. (5): the query has the
// keys' Kronecker form).
__device__ __forceinline__ float query_elem(const DecodeParams& P, int64_t row, int i, int j) {
    const kpa_dims& d = P.d;
    if (P.a_q == nullptr) return P.q[(row * (d.p1 * d.p2) + i) * (d.q1 * d.q2) + j];
    const int i1 = i / d.p2, i2 = i % d.p2, j1 = j / d.q2, j2 = j % d.q2;
    const float* a = P.a_q + ((row * P.r_q) * d.p1 + i1) * d.q1 + j1;
    const float* bb = P.b_q + ((row * P.r_q) * d.p2 + i2) * d.q2 + j2;
    float acc = 0.f;
    for (int r = 0; r < P.r_q; ++r) acc = fmaf(a[(int64_t)r * d.p1 * d.q1], bb[(int64_t)r * d.p2 * d.q2], acc);
    return acc / (float)P.r_q;
}

// Visible slots of query n of sequence b (causal: the n_q newest slots hold
// the queries' own tokens).  Out-of-range ctx_len is clamped and flagged.
__device__ __forceinline__ int visible_slots(const DecodeParams& P, int b, int n) {
    int ctx = P.ctx_len[b];
    if (ctx < 0 || ctx > P.max_ctx) {
        if (P.dev_status && n == 0 && threadIdx.x == 0) atomicOr(P.dev_status, (uint32_t)KPA_DEV_CTX_OUT_OF_RANGE);
        ctx = ctx < 0 ? 0 : P.max_ctx;
    }
    int vis = P.causal ? ctx - P.n_q + n + 1 : ctx;
    if (vis > ctx) vis = ctx;
    if (vis < 0) vis = 0;
    return vis;
}

// The chunk-0 workgroup of a row clears that row's merge counters; the merge
// kernel runs after the decode kernel on the same stream and leaves them at 0.
__device__ __forceinline__ void clear_merge_counters(const DecodeParams& P, int64_t row, int split) {
    if (P.merge_count && split == 0) {
        const int h = P.d.p1 * P.d.p2;
        for (int i = threadIdx.x; i < h; i += blockDim.x) P.merge_count[row * h + i] = 0u;
    }
}

// Events a decode launcher has the runtime stamp with its kernel's own start
// and end (hipExtLaunchKernel), for measurement; both null = plain launch.
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (one per translation unit).
hipError_t launch_append(const AppendParams& P, hipStream_t s);
hipError_t launch_project_append(const ProjectParams& P, hipStream_t s, const KernelEvents& ev);
hipError_t launch_decode_valu(const DecodeParams& P, hipStream_t s, const KernelEvents& ev);
hipError_t launch_merge(const DecodeParams& P, hipStream_t s);
hipError_t launch_stream_xor(const void* buf, int64_t bytes, uint32_t* partial, int n_blocks, hipStream_t s,
                             const KernelEvents& ev);
hipError_t launch_decode_mfma(const DecodeParams& P, hipStream_t s, const KernelEvents& ev);
bool decode_mfma_supported(const kpa_dims& d, int n_q);
int decode_mfma_blocks_per_cu(const kpa_dims& d, int n_q);
int decode_mfma_fill_pct(const kpa_dims& d, int n_q);  // percent of the resident slots the planner fills
int decode_valu_blocks_per_cu(const kpa_dims& d);
int decode_mfma_query_groups(const kpa_dims& d, int n_q);
// Multi-query decode with K and V rebuilt per tile on the matrix cores
// (decode_rebuild.hip): taken from kRebuildMinQ queries per sequence.
constexpr int kRebuildMinQ = 8;
// With the factors' roles swapped (q1 = 8, q2 = 16, p1 = 8): from 12.  A
// query group is 16 wide, so the rebuild costs about the same from 8 to 16
// queries while the factor-space kernel's time grows with them: on
// long_512k's split (8 x 16400 tokens) 8 queries take 137.0 us there
// against 160.9 rebuilt, 16 queries 250.4 against 175.3.
constexpr int kRebuildMinQSwapped = 12;
hipError_t launch_decode_rebuild(const DecodeParams& P, hipStream_t s, const KernelEvents& ev);
bool decode_rebuild_supported(const kpa_dims& d, int n_q);
int decode_rebuild_blocks_per_cu(const kpa_dims& d);
int decode_rebuild_head_groups(const kpa_dims& d);  // workgroups per chunk and query group
int decode_rebuild_query_groups(int n_q);

}  // namespace kpa
