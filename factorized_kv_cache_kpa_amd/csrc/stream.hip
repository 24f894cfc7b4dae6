// kpa_stream_xor kernel: a plain streaming read, the measured ceiling that
// the decode kernels' HBM rate is set against.  Each workgroup reads one
// contiguous share of the buffer once with 16-byte nontemporal loads, four
// in flight per thread (the decode kernels' own load form), and writes the
// XOR of the share's 32-bit words.
#include "kpa_common.hpp"
#include "kpa_mfma.hpp"

namespace kpa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ void __launch_bounds__(kStreamThreads) stream_xor_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                                     int64_t share16, uint32_t* partial) {
    const int64_t lo = (int64_t)blockIdx.x * share16;
    const int64_t hi = min(lo + share16, n16);
    constexpr int kRound = kStreamThreads * kStreamUnroll;
    const int64_t full = hi > lo ? lo + (hi - lo) / kRound * kRound : lo;  // end of the whole rounds
    uint32_t acc = 0;
    for (int64_t i = lo + threadIdx.x; i < full; i += kRound) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (int64_t i = full + threadIdx.x; i < hi; i += kStreamThreads) {  // the share's ragged end
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, x);
    __shared__ uint32_t wave_acc[kStreamThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kStreamThreads / 64; ++w) r ^= wave_acc[w];
        partial[blockIdx.x] = r;
    }
}

}  // namespace

hipError_t launch_stream_xor(const void* buf, int64_t bytes, uint32_t* partial, int n_blocks, hipStream_t s,
                             const KernelEvents& ev) {
    const int64_t n16 = bytes / 16;
    const int64_t share16 = (n16 + n_blocks - 1) / n_blocks;
    hipExtLaunchKernelGGL(stream_xor_kernel, dim3(n_blocks), dim3(kStreamThreads), 0, s, ev.start, ev.stop, 0,
                          static_cast<const u32x4*>(buf), n16, share16, partial);
    return hipGetLastError();
}

}  // namespace kpa
