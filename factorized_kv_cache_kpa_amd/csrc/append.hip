// kpa_cache_append kernels (B^K rotated at write time; the per-token work
// and its citations are in kpa_append.hpp).
//  * append_tile_kernel: one workgroup per (32-slot cache tile, sequence) the
//    new tokens touch.  The float64 angle of each (token, rotary pair index)
//    is computed once (a B^K row of every rank and head row shares it), the
//    feature-chunk sets are written as whole 16-byte chunks and the value
//    sets slot-contiguous.
//  * append_kernel: one workgroup per (new token, sequence); for decode-step
//    token counts, and for q2 > 64, whose angle table would not fit the tile
//    kernel's LDS.
// Both write the same bytes: the elements of the new tokens' slots and their
// positions (never the padding of a chunk), with the same float64 rotation.
#include "kpa_append.hpp"

namespace kpa {
namespace {

constexpr int kMaxTilePairs = 32;  // q2 / 2 the tile kernel's angle table holds
constexpr int64_t kPerTokenMax = 4096;  // new tokens (all sequences) for the per-token kernel
// input rows (bytes) the tile kernel stages in LDS: with the largest angle
// table (32 pairs: 32 KB) the launch stays within 64 KB of dynamic LDS
constexpr int kStageRowMax = 992;
static_assert(2 * kTileSlots * kMaxTilePairs * 8 + kTileSlots * (kStageRowMax + kChunkBytes) <= 65536,
              "the tile kernel's LDS fits 64 KB");
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

template <bool kF32>
__global__ void __launch_bounds__(256) append_kernel(AppendParams P) {
    append_token<kF32>(P.d, P.L, P.cache, P.capacity, P.in, P.dev_status, blockIdx.y, blockIdx.x, threadIdx.x,
                       blockDim.x);
}

__device__ __forceinline__ int floor_div32(int x) {
    return x >= 0 ? x / kTileSlots : -((-x + kTileSlots - 1) / kTileSlots);
}

template <bool kF32>
__global__ void __launch_bounds__(256) append_tile_kernel(AppendParams P) {
    using E = typename std::conditional<kF32, float, uint16_t>::type;
    constexpr int PC = kChunkBytes / (int)sizeof(E);  // elements per 16-byte chunk
    // LDS, sized by the launch for these dims: the angle table (cos, sin per
    // slot position and pair index), then the stage (32 rows of the longest
    // staged set, each padded by 16 bytes)
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ int pos_s[kTileSlots];
    __shared__ int ok_s[kTileSlots];
    const int half_pairs = P.d.q2 / 2;  // (at most kMaxTilePairs: the launch checks)
    double* const cs_tab = reinterpret_cast<double*>(dyn);
    double* const sn_tab = cs_tab + kTileSlots * half_pairs;
    uint8_t* const stage = dyn + 2 * kTileSlots * half_pairs * sizeof(double);
    const AppendInputs& in = P.in;
    const Layout& L = P.L;
    const int b = blockIdx.y;
    const int s0 = in.slot0[b];
    // in 64 bits: s0 comes from device memory and may sit near the int32 limit
    const int64_t tile = (int64_t)floor_div32(s0) + blockIdx.x;
    const int64_t base = tile * kTileSlots;  // slot of position 0 of this tile
    // new tokens n in [n_lo, n_hi) fall in this tile, at t = s0 + n - base
    const int n_lo = (int)max((int64_t)0, base - s0);
    const int n_hi = (int)min((int64_t)in.n_new, base + kTileSlots - s0);
    if (n_lo >= n_hi) return;
    const int tid = threadIdx.x;
    if (tid < kTileSlots) {
        const int n = (int)(base + tid - s0);
        const bool mine = n >= n_lo && n < n_hi;
        const int64_t slot = base + tid;
        const int pos = mine ? in.positions[(int64_t)b * in.n_new + n] : -1;
        const bool ok = mine && slot >= 0 && slot < P.capacity && pos >= 0;
        if (mine && !ok && P.dev_status) {
            uint32_t bits = 0;
            if (slot < 0 || slot >= P.capacity) bits |= KPA_DEV_SLOT_OUT_OF_RANGE;
            if (pos < 0) bits |= KPA_DEV_NEGATIVE_POSITION;
            atomicOr(P.dev_status, bits);
        }
        pos_s[tid] = pos;
        ok_s[tid] = ok;
    }
    __syncthreads();
    const int q2 = P.d.q2, half = q2 / 2;
    const double log2_base = log2((double)P.d.rope_base);
    for (int i = tid; i < kTileSlots * half; i += blockDim.x) {
        const int t = i / half, m = i % half;
        if (ok_s[t]) rope_angle(pos_s[t], m, q2, log2_base, sn_tab[t * half + m], cs_tab[t * half + m]);
    }
    __syncthreads();
    if (tile < 0 || tile >= L.n_tiles) return;  // (then no token of it is ok)
    uint8_t* tb = P.cache + ((int64_t)b * L.n_tiles + tile) * L.tile_bytes;
    const int64_t tok0 = (int64_t)b * in.n_new + (base - s0);  // token index of position 0 of the tile

    // The tile's tokens are consecutive rows of each input set.  A set whose
    // rows are whole 16-byte chunks (at most 1 KB), from a 16-byte aligned
    // input, is staged into LDS with coalesced 16-byte loads, one row per slot
    // position (rows padded by 16 bytes so that the readers spread over the
    // banks), then written out from there; any other set is read from global
    // memory element by element.  (Staging several sets per phase, or the
    // angles behind the first set's loads, measured slower.)
    const int t_lo = (int)(s0 + n_lo - base), n_t = n_hi - n_lo;
    auto stage_set = [&](const void* src_v, int ne) -> bool {
        const int row = ne * (int)sizeof(E);
        if (row % kChunkBytes != 0 || row > kStageRowMax || (reinterpret_cast<uintptr_t>(src_v) % kChunkBytes) != 0)
            return false;
        const uint8_t* src = static_cast<const uint8_t*>(src_v) + (tok0 + t_lo) * (int64_t)row;
        const int per_row = row / kChunkBytes;
        for (int i = tid; i < n_t * per_row; i += blockDim.x) {
            const int r = i / per_row, ch = i % per_row;
            *reinterpret_cast<u32x4_t*>(stage + (t_lo + r) * (row + kChunkBytes) + ch * kChunkBytes) =
                *reinterpret_cast<const u32x4_t*>(src + (int64_t)i * kChunkBytes);
        }
        return true;
    };

    // feature-chunk sets: A^K copied, B^K rotated; one (chunk, slot) per step
    for (int c = 0; c < 2; ++c) {
        const int ne = L.elems[c], nch = (ne + PC - 1) / PC;
        const void* srcv = c == 0 ? in.a_k : in.b_k;
        __syncthreads();  // the previous set's readers are done with the stage
        const bool staged = stage_set(srcv, ne);
        __syncthreads();
        const E* src = reinterpret_cast<const E*>(srcv);
        const E* st = reinterpret_cast<const E*>(stage);
        const int srow = ne + PC;  // staged row stride in elements
        for (int u = tid; u < nch * kTileSlots; u += blockDim.x) {
            const int cc = u / kTileSlots, t = u % kTileSlots;
            if (!ok_s[t]) continue;
            const int cnt = min(PC, ne - cc * PC);
            E v[PC];
            if (staged) {
                // whole chunks (the row is a multiple of 16 bytes)
                const u32x4_t w = *reinterpret_cast<const u32x4_t*>(st + t * srow + cc * PC);
                __builtin_memcpy(v, &w, sizeof(w));
            } else {
                const E* from = src + (tok0 + t) * ne + cc * PC;
#pragma unroll
                for (int k = 0; k < PC; ++k) v[k] = k < cnt ? from[k] : E(0);
            }
            if (c == 1) {
                // pairs (2j, 2j+1) of the chunk; a chunk starts on a pair (PC even)
#pragma unroll
                for (int k = 0; k < PC; k += 2) {
                    if (k >= cnt) break;
                    const int m = ((cc * PC + k) % q2) / 2;
                    double x0, x1;
                    if constexpr (kF32) {
                        x0 = v[k];
                        x1 = v[k + 1];
                    } else {
                        x0 = bf16_to_f32(v[k]);
                        x1 = bf16_to_f32(v[k + 1]);
                    }
                    double y0, y1;
                    rope_rotate(x0, x1, sn_tab[t * half + m], cs_tab[t * half + m], y0, y1);
                    if constexpr (kF32) {
                        v[k] = (float)y0;
                        v[k + 1] = (float)y1;
                    } else {
                        v[k] = f64_to_bf16_rne(y0);
                        v[k + 1] = f64_to_bf16_rne(y1);
                    }
                }
            }
            uint8_t* to = tb + L.off[c] + (int64_t)cc * (kTileSlots * kChunkBytes) + t * kChunkBytes;
            if (cnt == PC) {
                u32x4_t w;
                __builtin_memcpy(&w, v, sizeof(w));
                *reinterpret_cast<u32x4_t*>(to) = w;
            } else {
#pragma unroll
                for (int k = 0; k < PC; ++k)
                    if (k < cnt) store_elem<E>(to + k * sizeof(E), v[k]);
            }
        }
    }
    // value-format sets (A^V, B^V): element rows of 32 slots
    for (int c = 2; c < 4; ++c) {
        const int ne = L.elems[c];
        const void* srcv = c == 2 ? in.a_v : in.b_v;
        __syncthreads();
        const bool staged = stage_set(srcv, ne);
        __syncthreads();
        const E* src = reinterpret_cast<const E*>(srcv);
        const E* st = reinterpret_cast<const E*>(stage);
        const int srow = ne + PC;
        for (int u = tid; u < ne * kTileSlots; u += blockDim.x) {
            const int e = u / kTileSlots, t = u % kTileSlots;
            if (!ok_s[t]) continue;
            const E val = staged ? st[t * srow + e] : src[(tok0 + t) * ne + e];
            store_elem<E>(tb + L.off[c] + ((int64_t)e * kTileSlots + t) * sizeof(E), val);
        }
    }
    if (tid < kTileSlots && ok_s[tid]) {
        int32_t* positions = reinterpret_cast<int32_t*>(P.cache + L.positions_off);
        positions[(int64_t)b * L.n_tiles * kTileSlots + base + tid] = pos_s[tid];
    }
}

}  // namespace

hipError_t launch_append(const AppendParams& P, hipStream_t s) {
    // The tile kernel's chain of staged phases costs ~12-20 us even for one
    // token per sequence; up to kPerTokenMax new tokens in all, one block per
    // token is faster (decode steps: 5.6-7.1 us; the two break even at
    // 32 x 128 tokens) and writes the same bytes.
    if (P.d.q2 / 2 <= kMaxTilePairs && (int64_t)P.in.n_new * P.batch > kPerTokenMax) {
        // the new tokens of a sequence touch at most ceil(n_new / 32) + 1 tiles
        const dim3 grid((P.in.n_new + kTileSlots - 1) / kTileSlots + 1, P.batch);
        int row = 0;  // the longest row the kernel may stage
        for (int c = 0; c < 4; ++c) {
            const int r = P.L.elems[c] * P.L.elem_bytes;
            if (r % kChunkBytes == 0 && r <= kStageRowMax) row = r > row ? r : row;
        }
        const size_t lds = 2 * (size_t)kTileSlots * (P.d.q2 / 2) * sizeof(double) +
                           (size_t)kTileSlots * (row + kChunkBytes);
        if (P.d.dtype == KPA_F32)
            hipLaunchKernelGGL(append_tile_kernel<true>, grid, dim3(256), lds, s, P);
        else
            hipLaunchKernelGGL(append_tile_kernel<false>, grid, dim3(256), lds, s, P);
        return hipGetLastError();
    }
    const dim3 grid(P.in.n_new, P.batch);
    if (P.d.dtype == KPA_F32)
        hipLaunchKernelGGL(append_kernel<true>, grid, dim3(256), 0, s, P);
    else
        hipLaunchKernelGGL(append_kernel<false>, grid, dim3(256), 0, s, P);
    return hipGetLastError();
}

}  // namespace kpa
