// Register types and small helpers for the gfx950 matrix-core kernels.
//
// Operand layouts of the bf16 MFMA instructions used here (wave of 64 lanes):
//   v_mfma_f32_32x32x16_bf16: A[m][k] is element k%8 of lane m + 32*(k/8);
//     B[k][n] is element k%8 of lane n + 32*(k/8); D[m][n] is register
//     (m/8)*4 + m%4 of lane n + 32*((m/4)%2).
//   v_mfma_f32_16x16x32_bf16: A[m][k] is element k%8 of lane m + 16*(k/8);
//     B[k][n] is element k%8 of lane n + 16*(k/8); D[m][n] is register m%4
//     of lane n + 16*(m/4).
//   v_mfma_f32_4x4x4_16b_bf16: 16 independent 4x4x4 blocks, block b in lanes
//     4b .. 4b+3: A_b[i][k] is element k of lane 4b + i; B_b[k][j] is element
//     k of lane 4b + j; D_b[i][j] is register i of lane 4b + j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kpa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;  // 4 bf16: a 4x4x4 MFMA operand
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

template <typename T>
__device__ __forceinline__ T ld16(const uint8_t* p) {
    return __builtin_bit_cast(T, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

// 16-byte load with the nontemporal hint (`nt`): for cache bytes that one
// decode step reads once.  On MI355X a streaming read of a 768 MiB buffer
// reaches ~7.0 TB/s with the hint and ~6.1 TB/s without.
template <typename T>
__device__ __forceinline__ T ld16_nt(const uint8_t* p) {
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ bf16x8 ld_lds16(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void ld_lds32(const float* p, float* out) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[k] = a[k];
        out[4 + k] = b[k];
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ void unpack_bf16x4(uint2 u, float& a, float& b, float& c, float& d) {
    a = __uint_as_float(u.x << 16);
    b = __uint_as_float(u.x & 0xffff0000u);
    c = __uint_as_float(u.y << 16);
    d = __uint_as_float(u.y & 0xffff0000u);
}

__device__ __forceinline__ void unpack_bf16x8(bf16x8 v, float* out) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(u[k] << 16);
        out[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
}

typedef __attribute__((ext_vector_type(2))) float f32x2;

// Round 8 floats to bf16 (nearest even), two per v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2 * k], v[2 * k + 1]}, bf16x2));
    return __builtin_bit_cast(bf16x8, r);
}

// bf16 of two floats in one dword (low half = first), round to nearest even.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 2^x on the hardware exp unit (x <= 0 here; results below 2^-126 flush to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi).
__device__ __forceinline__ void split_bf16x8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const __bf16 h = (__bf16)v[k];
        hi[k] = h;
        lo[k] = (__bf16)(v[k] - (float)h);
    }
}

// The value of lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0] holds the lower half's value in every lane, r[1] the upper half's.
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// LDS byte address of a __shared__ pointer, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// One wave copies 64 x 16 B from global memory (each lane its own address)
// into LDS at [lds, lds + 1 KB) without passing through registers
// (global_load_lds_dwordx4; M0 holds the LDS base).  Completion is tracked by
// vmcnt; the caller waits with s_waitcnt vmcnt before reading the LDS bytes.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool kNT = false>
__device__ __forceinline__ void dma_to_lds16(const void* gaddr, uint32_t lds) {
    if constexpr (kNT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(gaddr)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gaddr)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// Make this wave's LDS writes visible to its other lanes (the wave's LDS
// operations complete in order; the fences keep the compiler from moving
// LDS accesses across this point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x(l) + x(l ^ 32) in every lane.
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace kpa
