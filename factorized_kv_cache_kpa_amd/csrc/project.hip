// kpa_project_append kernel: the factor projection of new tokens' hidden
// states as one GEMM on the matrix cores, its epilogue writing the factors
// straight into the tiled cache.
//
// [KPA] "Kronecker Product Attention: Memory-Efficient KV Compression via
//       Structured Factorization", Eq. (5) and the text after it: every
//       factor is a linear map of the token's hidden state, the ranks of a
//       factor type merged into one weight matrix whose product is reshaped to
//       [R][p][q].  Here the four merged matrices are stacked into one weight
//       (rows B^K, A^K, A^V, B^V), so one GEMM yields every factor of a token.
//       The cache then receives what kpa_cache_append would store (Thm. 2.4,
//       §2.5: only B^K rotated), except that B^K is rotated from the float32
//       products and every value is rounded once, to the cache type.
//
// Out[f][t] = sum_c W[f][c] x[t][c]: M = factor rows (f), N = tokens (t),
// K = d_model, bf16 operands with float32 accumulation
// (v_mfma_f32_32x32x16_bf16).  One workgroup per 32 rows x 32 tokens; its NW
// waves (4, 8 or 16: as many as d_model allows, so that more loads of the
// weight are in flight) split d_model NW ways and add their partial tiles
// through LDS.  In
// the accumulator layout a lane holds one token and, for register r, row
// 8 (r / 4) + 4 (lane / 32) + r % 4: the two features of a RoPE pair (even,
// odd) sit in neighbouring registers of one lane.
#include "kpa_append.hpp"
#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace {

// Epilogue shared by both kernels: four consecutive stacked rows fb .. fb+3
// (fb a multiple of 4) of one token (sequence b, cache slot `slot`, position
// pos) go to the cache.  Stacked rows: B^K [0, n1), A^K [n1, n10), A^V
// [n10, n102), B^V [n102, F).  A B^K row pair (even, odd) is rotated in
// float64 ([KPA] Def. 2.3) and every value is rounded once to the cache type.
// The recorder lane (one per token) writes the position and reports a slot
// out of range or a negative position; such a token is not stored.
template <bool kF32>
__device__ __forceinline__ void store_rows4(const ProjectParams& P, int b, int slot, int pos, int fb, const float* v,
                                            bool recorder) {
    if (slot < 0 || slot >= P.capacity || pos < 0) {
        if (recorder && P.dev_status) {
            uint32_t bits = 0;
            if (slot < 0 || slot >= P.capacity) bits |= KPA_DEV_SLOT_OUT_OF_RANGE;
            if (pos < 0) bits |= KPA_DEV_NEGATIVE_POSITION;
            atomicOr(P.dev_status, bits);
        }
        return;
    }
    const Layout& L = P.L;
    const int F = P.n_feat;
    uint8_t* tile_base = P.cache + ((int64_t)b * L.n_tiles + slot / kTileSlots) * L.tile_bytes;
    const int ts = slot % kTileSlots;
    const int n1 = L.elems[1], n10 = n1 + L.elems[0], n102 = n10 + L.elems[2];
    const int q2 = P.d.q2;
    const double log2_base = log2((double)P.d.rope_base);
    auto put = [&](int c, int e, float val) {
        if constexpr (kF32)
            store_elem<float>(tile_base + elem_offset(L, c, e, ts), val);
        else
            store_elem<uint16_t>(tile_base + elem_offset(L, c, e, ts), f32_to_bf16_rne(val));
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int fr = fb + j;
        if (fr >= F) break;
        if (fr < n1) {
            // B^K: rows fr (even) and fr + 1 form one RoPE pair (n1 is even)
            if (j % 2 == 0) {
                double y0, y1;
                rope_pair((double)v[j], (double)v[j + 1], pos, (fr % q2) / 2, q2, log2_base, y0, y1);
                if constexpr (kF32) {
                    store_elem<float>(tile_base + elem_offset(L, 1, fr, ts), (float)y0);
                    store_elem<float>(tile_base + elem_offset(L, 1, fr + 1, ts), (float)y1);
                } else {
                    store_elem<uint16_t>(tile_base + elem_offset(L, 1, fr, ts), f64_to_bf16_rne(y0));
                    store_elem<uint16_t>(tile_base + elem_offset(L, 1, fr + 1, ts), f64_to_bf16_rne(y1));
                }
            }
        } else if (fr < n10) {
            put(0, fr - n1, v[j]);
        } else if (fr < n102) {
            put(2, fr - n10, v[j]);
        } else {
            put(3, fr - n102, v[j]);
        }
    }
    if (recorder) {
        int32_t* positions = reinterpret_cast<int32_t*>(P.cache + L.positions_off);
        positions[(int64_t)b * L.n_tiles * kTileSlots + slot] = pos;
    }
}

template <bool kF32, int NW>
__global__ void __launch_bounds__(NW * 64) project_append_kernel(ProjectParams P) {
    __shared__ float part[NW][16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int F = P.n_feat, M = P.n_tok, K = P.d_model;
    const int f = blockIdx.x * 32 + l32;  // A-operand row of this lane
    const int t = blockIdx.y * 32 + l32;  // B-operand column (token) of this lane
    const bool f_ok = f < F, t_ok = t < M;
    const uint8_t* wrow = reinterpret_cast<const uint8_t*>(P.w + (int64_t)(f_ok ? f : 0) * K);
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(P.x + (int64_t)(t_ok ? t : 0) * K);
    const int kq = K / NW;  // a multiple of 16 (the launcher picks NW so)
    // the lane's token for the epilogue (column blockIdx.y * 32 + lane % 32):
    // its slot and position are read now, their latency hidden by the GEMM
    const int tok = t;
    const int tb = t_ok ? tok / P.n_new : 0, tn = t_ok ? tok % P.n_new : 0;
    const int slot = t_ok ? slot_add(P.slot0[tb], tn) : -1;
    const int pos = t_ok ? P.positions[tok] : -1;
    const int k0 = wave * kq;
    // The K order inside each block of 64 is permuted (the same for both
    // operands, so the sums are unchanged): in MFMA step s of a block, lane
    // (m, hi) supplies elements 32 hi + 8 s .. + 7, so over the block's four
    // steps each lane reads 64 contiguous bytes and each row is read as whole
    // 128-byte lines (a tail shorter than 128 keeps the plain order: lane
    // (m, hi) supplies elements 8 hi .. 8 hi + 7 of the step).  Operands of KU steps are loaded before any of them is
    // used (every load in flight at once: at decode-sized token counts there
    // are few workgroups); two accumulators so consecutive products do not
    // wait for each other.  Rows past F and tokens past the end read row 0 /
    // token 0: their products land in outputs the epilogue never stores.
    constexpr int KU = 8;  // two blocks of 64
    f32x16 acc0 = {}, acc1 = {};
    int k = k0;
    for (; k + 16 * KU <= k0 + kq; k += 16 * KU) {
        bf16x8 a[KU], bm[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int e = k + 64 * (u / 4) + 32 * hi + 8 * (u % 4);
            a[u] = ld16<bf16x8>(wrow + (int64_t)e * 2);
            bm[u] = ld16<bf16x8>(xrow + (int64_t)e * 2);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the first product
#pragma unroll
        for (int u = 0; u < KU; u += 2) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], bm[u], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u + 1], bm[u + 1], acc1, 0, 0, 0);
        }
    }
    for (; k < k0 + kq; k += 16) {  // the rest, one step at a time in the plain K order
        const int e = k + 8 * hi;
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16<bf16x8>(wrow + (int64_t)e * 2),
                                                     ld16<bf16x8>(xrow + (int64_t)e * 2), acc0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave][r][lane] = acc0[r] + acc1[r];
    __syncthreads();

    // waves 0 .. 3 finish: wave w takes registers 4w .. 4w+3 of every lane,
    // rows 8w + 4hi + j
    if (wave >= 4) return;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += part[w][4 * wave + j][lane];
        v[j] = s;
    }
    if (!t_ok) return;
    // one lane per token reports and records (the workgroup of the first rows)
    store_rows4<kF32>(P, tb, slot, pos, blockIdx.x * 32 + 8 * wave + 4 * hi, v,
                      blockIdx.x == 0 && wave == 0 && hi == 0);
}

// Prefill-sized token counts: an LDS-tiled GEMM.  One workgroup (4 waves)
// computes 128 stacked rows x 128 tokens, d_model in steps of 64.  Each step's
// operands (128 weight rows and 128 token rows of 64 bf16, 16 KB each) go
// HBM -> LDS by direct DMA, double-buffered, one step ahead; wave (wm, wn)
// then multiplies its 64 x 64 quarter as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, operands read from LDS.  In LDS a row is 128 B
// (eight 16-byte chunks); chunk c of row r sits at position c ^ ((r >> 1) & 7)
// so that the 32 rows one operand read touches spread over the banks (the
// DMA lane that fills a position fetches the chunk that belongs there).
// Rows past F and tokens past the end read the last valid row; their
// outputs are not stored.  The epilogue is the small kernel's.
constexpr int kTB = 128;   // rows and tokens per workgroup
constexpr int kTK = 64;    // d_model per step
constexpr int kTileOpBytes = kTB * kTK * 2;
constexpr int kTiledMinTokens = 1024;
constexpr int kXcdCount = 8;  // MI355X: workgroups dealt to 8 XCDs round-robin

template <bool kF32>
__global__ void __launch_bounds__(256, 2) project_tiled_kernel(ProjectParams P) {
    // two steps' operands; after the GEMM, the 128 x 128 float32 result tile
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kTileOpBytes];
    uint8_t* const sa0 = lds;
    uint8_t* const sa1 = lds + kTileOpBytes;
    uint8_t* const sb0 = lds + 2 * kTileOpBytes;
    uint8_t* const sb1 = lds + 3 * kTileOpBytes;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const int F = P.n_feat, T = P.n_tok, K = P.d_model;
    // Workgroup -> (row tile, token tile), XCD-aware: the hardware deals
    // workgroup L to XCD L % 8, and XCD x takes a contiguous range of the work
    // items, token tile major, row tile minor.  The row tiles of one token
    // tile then run side by side on one XCD and read its token rows through
    // that XCD's L2, not once per row tile from HBM.
    const int n_rt = (F + kTB - 1) / kTB, n_tt = (T + kTB - 1) / kTB;
    const int total = n_rt * n_tt, xcd = blockIdx.x % kXcdCount, k_in = blockIdx.x / kXcdCount;
    const int item = xcd * (total / kXcdCount) + min(xcd, total % kXcdCount) + k_in;
    const int f0 = (item % n_rt) * kTB, t0 = (item / n_rt) * kTB;

    // DMA plan: 16 instructions of 1 KB per operand and step, 4 per wave; the
    // instruction d fills rows 8d .. 8d+7, lane i row 8d + i/8, position i%8
    const uint8_t* arow[4];
    const uint8_t* brow[4];
    int chunk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int d = wave * 4 + u, r = 8 * d + (lane >> 3);
        chunk[u] = (lane & 7) ^ ((r >> 1) & 7);
        arow[u] = reinterpret_cast<const uint8_t*>(P.w + (int64_t)min(f0 + r, F - 1) * K);
        brow[u] = reinterpret_cast<const uint8_t*>(P.x + (int64_t)min(t0 + r, T - 1) * K);
    }
    auto issue = [&](int k0, uint8_t* sa, uint8_t* sb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int d = wave * 4 + u;
            dma_to_lds16(arow[u] + (int64_t)k0 * 2 + chunk[u] * 16, lds_addr(sa + d * 1024));
            dma_to_lds16(brow[u] + (int64_t)k0 * 2 + chunk[u] * 16, lds_addr(sb + d * 1024));
        }
    };

    // the epilogue's token of this thread (t0 + threadIdx.x % 128): its slot
    // and position are read now, their latency hidden by the GEMM
    const int tk = threadIdx.x % kTB, t_ep = t0 + tk;
    const bool t_ok = t_ep < T;
    const int tb = t_ok ? t_ep / P.n_new : 0;
    const int slot = t_ok ? slot_add(P.slot0[tb], t_ep % P.n_new) : -1;
    const int pos = t_ok ? P.positions[t_ep] : -1;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    // operand reads: row m of a block, chunk kc (0 .. 7) of the step
    auto rd = [&](const uint8_t* buf, int m, int kc) {
        return ld_lds16(reinterpret_cast<const uint16_t*>(buf + m * 128 + ((kc ^ ((m >> 1) & 7)) * 16)));
    };
    // The whole step's operands are read first (16 reads, 64 registers), so
    // the LDS latency of a later K slice hides behind the earlier slices'
    // MFMAs instead of stalling every slice.
    auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
        bf16x8 a[kTK / 16][2], bv[kTK / 16][2];
#pragma unroll
        for (int kk = 0; kk < kTK / 16; ++kk) {
            const int kc = 2 * kk + hi;  // this lane's 8 of the step's 16
#pragma unroll
            for (int i = 0; i < 2; ++i) a[kk][i] = rd(sa, wm * 64 + 32 * i + l32, kc);
#pragma unroll
            for (int j = 0; j < 2; ++j) bv[kk][j] = rd(sb, wn * 64 + 32 * j + l32, kc);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
        for (int kk = 0; kk < kTK / 16; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], bv[kk][j], acc[i][j], 0, 0, 0);
    };
    // One exit from the K loop (the step's buffers chosen by its parity), so
    // the accumulators stay in the same registers throughout.
    const int nk = K / kTK;
    issue(0, sa0, sb0);
    for (int kt = 0; kt < nk; ++kt) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this step's DMA
        __syncthreads();                     // ... every wave's; the other buffers are free
        const bool odd = kt & 1;
        if (kt + 1 < nk) issue((kt + 1) * kTK, odd ? sa0 : sa1, odd ? sb0 : sb1);
        compute(odd ? sa1 : sa0, odd ? sb1 : sb0);
    }

    // epilogue through LDS: block (i, j) register r holds row 32 i + 8 (r / 4)
    // + 4 hi + r % 4 of the wave's quarter, for token column 32 j + lane % 32
    __syncthreads();  // every wave is done with the last step's operands
    float* const tile = reinterpret_cast<float*>(lds);  // [128 rows][128 tokens]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                tile[(wm * 64 + 32 * i + 8 * (r / 4) + 4 * hi + r % 4) * kTB + wn * 64 + 32 * j + l32] = acc[i][j][r];
    __syncthreads();
    if (!t_ok) return;
    // each thread: its token, row groups 4g .. 4g+3 for g = threadIdx.x / 128, +2, ...
#pragma unroll 1
    for (int g = threadIdx.x / kTB; g < kTB / 4; g += 256 / kTB) {
        const int fb = f0 + 4 * g;
        if (fb >= F) break;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = tile[(4 * g + r) * kTB + tk];
        store_rows4<kF32>(P, tb, slot, pos, fb, v, f0 == 0 && g == 0);
    }
}

template <int NW>
void launch_nw(const ProjectParams& P, hipStream_t s, const KernelEvents& ev) {
    dim3 grid((P.n_feat + 31) / 32, (P.n_tok + 31) / 32);
    if (P.d.dtype == KPA_F32)
        hipExtLaunchKernelGGL((project_append_kernel<true, NW>), grid, dim3(NW * 64), 0, s, ev.start, ev.stop, 0, P);
    else
        hipExtLaunchKernelGGL((project_append_kernel<false, NW>), grid, dim3(NW * 64), 0, s, ev.start, ev.stop, 0, P);
}

}  // namespace

// d_model is a multiple of 64; each wave's share must be a multiple of 16.
// From 1024 tokens on, the LDS-tiled kernel (a 128 x 128 tile per
// workgroup); below, the small kernel, whose 32 x 32 tiles give enough
// workgroups at decode-step token counts.
hipError_t launch_project_append(const ProjectParams& P, hipStream_t s, const KernelEvents& ev) {
    if (P.n_tok >= kTiledMinTokens) {
        const dim3 grid(((P.n_feat + kTB - 1) / kTB) * ((P.n_tok + kTB - 1) / kTB));
        if (P.d.dtype == KPA_F32)
            hipExtLaunchKernelGGL(project_tiled_kernel<true>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, P);
        else
            hipExtLaunchKernelGGL(project_tiled_kernel<false>, grid, dim3(256), 0, s, ev.start, ev.stop, 0, P);
        return hipGetLastError();
    }
    if (P.d_model % (16 * 16) == 0 && P.d_model >= 1024)
        launch_nw<16>(P, s, ev);
    else if (P.d_model % (8 * 16) == 0 && P.d_model >= 512)
        launch_nw<8>(P, s, ev);
    else
        launch_nw<4>(P, s, ev);
    return hipGetLastError();
}

}  // namespace kpa
