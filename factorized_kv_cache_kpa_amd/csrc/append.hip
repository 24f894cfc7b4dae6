// kpa_cache_append kernel: one block per (new token, sequence) writes the
// token's factors into the tiled cache (B^K rotated at write time; the
// per-token work and its citations are in kpa_append.hpp).
#include "kpa_append.hpp"

namespace kpa {
namespace {

template <bool kF32>
__global__ void __launch_bounds__(256) append_kernel(AppendParams P) {
    append_token<kF32>(P.d, P.L, P.cache, P.capacity, P.in, P.dev_status, blockIdx.y, blockIdx.x, threadIdx.x,
                       blockDim.x);
}

}  // namespace

hipError_t launch_append(const AppendParams& P, hipStream_t s) {
    dim3 grid(P.in.n_new, P.batch);
    if (P.d.dtype == KPA_F32)
        hipLaunchKernelGGL(append_kernel<true>, grid, dim3(256), 0, s, P);
    else
        hipLaunchKernelGGL(append_kernel<false>, grid, dim3(256), 0, s, P);
    return hipGetLastError();
}

}  // namespace kpa
