// Shared device helpers for the gfx950 kernels: element types, bf16 packing,
// MFMA fragment types and the XCD-aware block remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdaconv {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---- scalar conversions ---------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 pair -> packed bf16 pair (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct ElemIO;

template <> struct ElemIO<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static void store(float *p, float x) { *p = x; }
};

template <> struct ElemIO<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p) { return (float)*p; }
    __device__ __forceinline__ static void store(bf16_t *p, float x) { *p = (bf16_t)x; }
};

// ---- barriers -----------------------------------------------------------------
// Workgroup barrier ordering LDS only.  __syncthreads() also drains this wave's
// outstanding global loads and stores (on gfx9 they share one counter), which
// would throw away any prefetch in flight; phases that hand data over through
// LDS only need this wave's LDS operations complete before the meeting point.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vector memory left in flight
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Fourth descriptor word of a raw (untyped, stride 0) buffer resource on gfx9.
constexpr int kBufWord3 = 0x00020000;

// ---- XCD-aware block remap --------------------------------------------------
// Workgroups are dealt round-robin over the 8 XCDs (each with its own L2).
// Remap the hardware block id so that every XCD receives a contiguous range
// of logical blocks; neighbouring logical blocks then share that XCD's L2.
// The map is a bijection on [0, nblocks).
__device__ __forceinline__ int xcd_remap(int hw_block, int nblocks) {
    const int nx = 8;
    const int q = nblocks / nx, r = nblocks % nx;
    const int xcd = hw_block % nx, i = hw_block / nx;
    return xcd * q + (xcd < r ? xcd : r) + i;
}

}  // namespace kdaconv
