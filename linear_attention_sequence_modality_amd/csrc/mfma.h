// MFMA fragment abstraction for gfx950.
//
// A fragment is the 8 values one lane contributes to a 16x16 output tile per
// 32-deep contraction step.  For v_mfma_f32_16x16x32_bf16 lane l supplies
// row (A) or column (B) l%16 and lane group g = l/16 supplies 8 k-slots;
// the fp32 path issues eight v_mfma_f32_16x16x4_f32, where instruction i
// consumes slot i of every lane, so the same fragment covers the same 32
// k-indices.  Which logical k sits in which (g, slot) is chosen by the
// loader; A and B only have to agree.  The 16x16 fp32 result holds, in lane
// l, rows 4*(l/16)+i (i = 0..3) of column l%16.
#pragma once

#include "common.h"

namespace kdaconv {

template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
    bf16x8_t v;
    __device__ __forceinline__ static Frag zero() {
        Frag f;
        f.v = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        return f;
    }
    // 8 consecutive elements (16-byte aligned)
    __device__ __forceinline__ static Frag ld8(const bf16_t *p) {
        Frag f;
        f.v = *reinterpret_cast<const bf16x8_t *>(p);
        return f;
    }
    // elements p0[0..3] then p1[0..3] (each 8-byte aligned)
    __device__ __forceinline__ static Frag ld4x2(const bf16_t *p0, const bf16_t *p1) {
        const uint2 a = *reinterpret_cast<const uint2 *>(p0);
        const uint2 b = *reinterpret_cast<const uint2 *>(p1);
        Frag f;
        uint4 u = make_uint4(a.x, a.y, b.x, b.y);
        f.v = __builtin_bit_cast(bf16x8_t, u);
        return f;
    }
    // four element pairs p[0..1], p[s..s+1], p[2s..], p[3s..] (4-byte aligned)
    __device__ __forceinline__ static Frag ld_pairs(const bf16_t *p, int s) {
        uint4 u;
        u.x = *reinterpret_cast<const uint32_t *>(p);
        u.y = *reinterpret_cast<const uint32_t *>(p + s);
        u.z = *reinterpret_cast<const uint32_t *>(p + 2 * s);
        u.w = *reinterpret_cast<const uint32_t *>(p + 3 * s);
        Frag f;
        f.v = __builtin_bit_cast(bf16x8_t, u);
        return f;
    }
    // eight single elements p[0], p[s], ..., p[7s]
    __device__ __forceinline__ static Frag ld_strided(const bf16_t *p, int s) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = p[i * s];
        return f;
    }
    __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
    __device__ __forceinline__ void set(int i, float x) { v[i] = (bf16_t)x; }
    __device__ __forceinline__ void st8(bf16_t *p) const {
        *reinterpret_cast<bf16x8_t *>(p) = v;
    }
};

template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ static Frag zero() {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
        return f;
    }
    __device__ __forceinline__ static Frag ld8(const float *p) {
        Frag f;
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
        return f;
    }
    __device__ __forceinline__ static Frag ld4x2(const float *p0, const float *p1) {
        Frag f;
        const float4 a = *reinterpret_cast<const float4 *>(p0);
        const float4 b = *reinterpret_cast<const float4 *>(p1);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
        return f;
    }
    __device__ __forceinline__ static Frag ld_pairs(const float *p, int s) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float2 a = *reinterpret_cast<const float2 *>(p + j * s);
            f.v[2 * j] = a.x;
            f.v[2 * j + 1] = a.y;
        }
        return f;
    }
    __device__ __forceinline__ static Frag ld_strided(const float *p, int s) {
        Frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.v[i] = p[i * s];
        return f;
    }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
    __device__ __forceinline__ void set(int i, float x) { v[i] = x; }
    __device__ __forceinline__ void st8(float *p) const {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ f32x4_t mma(const Frag<bf16_t> &a, const Frag<bf16_t> &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma(const Frag<float> &a, const Frag<float> &b, f32x4_t c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
    return c;
}

// One fp32 16x16x4 step: lane l supplies A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ f32x4_t mma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Store / load 4 consecutive elements of type T from fp32 values.
template <typename T> __device__ __forceinline__ void st4(T *p, const float (&x)[4]);
template <> __device__ __forceinline__ void st4<bf16_t>(bf16_t *p, const float (&x)[4]) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
template <> __device__ __forceinline__ void st4<float>(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <typename T> __device__ __forceinline__ void ld4(const T *p, float (&x)[4]);
template <> __device__ __forceinline__ void ld4<bf16_t>(const bf16_t *p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
}
template <> __device__ __forceinline__ void ld4<float>(const float *p, float (&x)[4]) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
}

// Load / store 8 consecutive elements of type T as fp32.
template <typename T> __device__ __forceinline__ void ld8f(const T *p, float (&x)[8]);
template <> __device__ __forceinline__ void ld8f<bf16_t>(const bf16_t *p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}
template <> __device__ __forceinline__ void ld8f<float>(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <typename T> __device__ __forceinline__ void st8f(T *p, const float (&x)[8]);
template <> __device__ __forceinline__ void st8f<bf16_t>(bf16_t *p, const float (&x)[8]) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}
template <> __device__ __forceinline__ void st8f<float>(float *p, const float (&x)[8]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
// A pair of elements (one 4-byte bf16 pair or one 8-byte fp32 pair).
template <typename T> __device__ __forceinline__ void st2(T *p, float a, float b);
template <> __device__ __forceinline__ void st2<bf16_t>(bf16_t *p, float a, float b) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
}
template <> __device__ __forceinline__ void st2<float>(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}

}  // namespace kdaconv
