// Chunk workspace layout shared by the chunk transform (kda.hip) and the
// state passes (kda_scan.hip), plus the small register helpers both use.
//
// One record per (head, chunk of 64 tokens), head-major over all chunks of
// the call.  Every field is stored in the register-fragment order in which the
// state passes consume it, so a lane of a consuming wave loads 16 contiguous
// bytes per fragment.
#pragma once

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace kdaconv {

constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// ---- workspace layout (per batch, head, chunk; element type T) ---------------
// Fragment order: kernel-2 lane l loads 16 contiguous bytes per fragment.
// dk-indexed fragments (W, Qt) hold, in slots 0..3 and 4..7, the channels
// 32ks + 4g + i and 32ks + 16 + 4g + i (g = l/16), matching the rows kernel 2
// holds of its state tiles 2ks and 2ks+1; token-indexed fragments (BT, Kh^T)
// are ordered likewise over tokens.
template <typename T, int DK, int DV>
struct Ws {
    static constexpr size_t W = 0;                 // [4 R][DK/32][64][8]  W rows of block R
    static constexpr size_t QT = W + 64 * DK;      // [4 R][DK/32][64][8]  Qt
    static constexpr size_t KH = QT + 64 * DK;     // [DK/16][2][64][8]    Kh^T (dk rows x tokens, k order as BT)
    static constexpr size_t BT = KH + 64 * DK;     // [4 R][2][64][8]      Bq rows of block R
    static constexpr size_t U = BT + 64 * 64;      // [DV/16][64][4 R][4]  Ut, accumulator order
    static constexpr size_t ELEMS = U + 64 * DV;
    static constexpr size_t GAM_BYTE = round_up(ELEMS * sizeof(T), 16);   // fp32 [DK], gam_pos order
    static constexpr size_t BYTES = round_up(GAM_BYTE + DK * sizeof(float), 256);
};

// Position of key channel c = 16 dt + 4 g + i in the stored chunk decay: the
// 4 DK/16 values a state-pass lane group g needs are contiguous, 2 per lane.
template <int DK> __device__ __forceinline__ int gam_pos(int c) {
    return ((c >> 2) & 3) * (DK / 4) + 4 * (c >> 4) + (c & 3);
}

// ---- raw 8-element rows (register prefetch without conversion) --------------
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16_t *p) { u = *reinterpret_cast<const uint4 *>(p); }
    // 8 elements at byte offset off of a buffer resource
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, unsigned off) {
        u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    // fp32 values rounded to bf16 (nearest even)
    __device__ __forceinline__ void set(const float (&x)[8]) {
        u = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                       pack_bf16x2(x[6], x[7]));
    }
    __device__ __forceinline__ void zero() { u = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void get(float (&x)[8]) const {
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
        x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, unsigned off) {
        a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u, 0, 0));
    }
    __device__ __forceinline__ void set(const float (&x)[8]) {
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(x[4], x[5], x[6], x[7]);
    }
    __device__ __forceinline__ void get(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

// Lane N of the calling lane's row of 16 (DPP row_newbcast).
template <int N> __device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, false));
}
// Run-time lane index; folds to one DPP operand once n is a constant after unrolling.
__device__ __forceinline__ float row_bcast(float x, int n) {
    switch (n) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
    }
}

template <typename T> __device__ __forceinline__ Frag<T> tiles_to_frag(const f32x4_t &lo, const f32x4_t &hi);
template <> __device__ __forceinline__ Frag<bf16_t> tiles_to_frag<bf16_t>(const f32x4_t &lo, const f32x4_t &hi) {
    const uint4 u = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                               pack_bf16x2(hi[2], hi[3]));
    Frag<bf16_t> f;
    f.v = __builtin_bit_cast(bf16x8_t, u);
    return f;
}
template <> __device__ __forceinline__ Frag<float> tiles_to_frag<float>(const f32x4_t &lo, const f32x4_t &hi) {
    Frag<float> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = lo[i];
        f.v[4 + i] = hi[i];
    }
    return f;
}

// Raw buffer loads: a lane-dependent offset plus a wave-uniform one.
template <typename T> struct BufLd;
template <> struct BufLd<bf16_t> {
    __device__ __forceinline__ static Frag<bf16_t> frag(__amdgpu_buffer_rsrc_t r, unsigned v, unsigned s) {
        Frag<bf16_t> f;
        f.v = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
        return f;
    }
    __device__ __forceinline__ static void raw8(Raw8<bf16_t> &x, __amdgpu_buffer_rsrc_t r, unsigned v, unsigned s) {
        x.u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
    }
};
template <> struct BufLd<float> {
    __device__ __forceinline__ static Frag<float> frag(__amdgpu_buffer_rsrc_t r, unsigned v, unsigned s) {
        const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0);
        const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, v, s + 16, 0);
        Frag<float> f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.v[i] = __uint_as_float(a[i]);
            f.v[4 + i] = __uint_as_float(b[i]);
        }
        return f;
    }
    __device__ __forceinline__ static void raw8(Raw8<float> &x, __amdgpu_buffer_rsrc_t r, unsigned v, unsigned s) {
        x.a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, 0));
        x.b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s + 16, 0));
    }
};

// An empty asm that reads and rewrites x: the value is computed before this
// point, so the compiler cannot sink the computation towards a later use.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x4_t &x) { asm volatile("" : "+v"(x)); }

// Instantiations of a launcher FN<T, DK, DV>(a, stream) for the supported
// head sizes and element types.
#define KDA_DISPATCH(FN)                                                                           \
    if (a.B == 0 || seq_chk0(a, a.B) == 0) return hipSuccess;                                      \
    if (bf16) {                                                                                    \
        if (a.dk == 64 && a.dv == 64) return FN<bf16_t, 64, 64>(a, stream);                        \
        if (a.dk == 64 && a.dv == 128) return FN<bf16_t, 64, 128>(a, stream);                      \
        if (a.dk == 128 && a.dv == 64) return FN<bf16_t, 128, 64>(a, stream);                      \
        if (a.dk == 128 && a.dv == 128) return FN<bf16_t, 128, 128>(a, stream);                    \
    } else {                                                                                       \
        if (a.dk == 64 && a.dv == 64) return FN<float, 64, 64>(a, stream);                         \
        if (a.dk == 64 && a.dv == 128) return FN<float, 64, 128>(a, stream);                       \
        if (a.dk == 128 && a.dv == 64) return FN<float, 128, 64>(a, stream);                       \
        if (a.dk == 128 && a.dv == 128) return FN<float, 128, 128>(a, stream);                     \
    }                                                                                              \
    return hipErrorInvalidValue;

}  // namespace kdaconv
