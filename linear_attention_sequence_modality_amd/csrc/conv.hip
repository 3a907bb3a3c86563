// Modality-aware depthwise short convolution (gfx950).
//
// Chimera pages: the conv runs before every KDA update, separately per
// modality -- a causal 1D depthwise conv over text tokens and a depthwise 3D
// conv over the visual tokens on their (t, h, w) grid (rainbus "core method";
// genai-atlas "How it works").  Taps: text 4 (last tap on the current token),
// visual 3x3x3 with zero padding; time offset P = 1 (symmetric) or 2 (causal).
//
// Design.  A depthwise conv has no channel contraction, so there is no
// matrix-core work: 27 multiply-adds per output against 2 bytes in and 2 out
// make the visual conv VALU-bound on fp32 vector units.  So:
//   * one wave owns one (stream, batch, h row, run of WR w positions, 128
//     channels) item and marches over t; lane l owns channels 2l, 2l+1.  All
//     addressing and every boundary test is wave-uniform: loads and stores are
//     raw buffer operations whose token offset is a scalar register, and a
//     lane only supplies its constant channel offset;
//   * each input slice is loaded once (3 rows x (WR+2) positions, one dword
//     per lane = 256 contiguous bytes per wave per token) and feeds the three
//     output slices t-1, t, t+1 from a 3-deep accumulator ring whose slot
//     index is static after unrolling the march by 3;
//   * bf16: the loaded dword (channel pair c, c+1 of one token) goes
//     unconverted into v_dot2_f32_bf16 against the weight pairs (w_c, 0) and
//     (0, w_c+1): one exact product and fp32 accumulation per instruction, no
//     bf16 -> fp32 unpacking.  fp32 streams use plain fma;
//   * blocks are remapped so each XCD works on a contiguous range of rows,
//     keeping the h-1/h/h+1 halo rows in that XCD's L2;
//   * text tokens form a separate block range: a wave slides the 4-tap causal
//     window over TR consecutive text tokens.
#include "common.h"
#include "launch.h"

namespace kdaconv {
namespace {

constexpr int WR = 8;     // w positions per wave item
constexpr int TR = 16;    // text tokens per wave item
constexpr int NT = 256;   // threads per block (4 waves)
constexpr int LANES = 64;
constexpr int CPW = 2 * LANES;   // channels per wave item

// Fourth descriptor word of a raw (untyped, stride 0) buffer resource on gfx9.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T> struct Ops;

template <> struct Ops<bf16_t> {
    typedef uint32_t XT;   // raw channel pair of one token
    struct Taps {
        uint32_t w[27][2];   // (w_c, 0) and (0, w_c+1) as bf16 pairs
    };
    __device__ __forceinline__ static void load_taps(Taps &tp, const bf16_t *wv, int c0, bool ok) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(wv);
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            tp.w[tap][0] = ok ? (uint32_t)p[(size_t)c0 * 27 + tap] : 0u;
            tp.w[tap][1] = ok ? (uint32_t)p[(size_t)(c0 + 1) * 27 + tap] << 16 : 0u;
        }
    }
    __device__ __forceinline__ static XT load(const char *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ __forceinline__ static XT bload(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    __device__ __forceinline__ static void bstore(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                                  float a, float b) {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), r, voff, soff, 0);
    }
    __device__ __forceinline__ static XT zero() { return 0u; }
    __device__ __forceinline__ static void mac(const Taps &tp, int tap, XT x, float &a0, float &a1) {
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                             __builtin_bit_cast(bf16x2_t, tp.w[tap][0]), a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                             __builtin_bit_cast(bf16x2_t, tp.w[tap][1]), a1, false);
    }
    __device__ __forceinline__ static void store(char *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
    __device__ __forceinline__ static float lo(XT x) { return bf16_lo(x); }
    __device__ __forceinline__ static float hi(XT x) { return bf16_hi(x); }
    __device__ __forceinline__ static float tapw(const bf16_t *w, size_t i) { return (float)w[i]; }
};

template <> struct Ops<float> {
    typedef float2 XT;
    struct Taps {
        float w[27][2];
    };
    __device__ __forceinline__ static void load_taps(Taps &tp, const float *wv, int c0, bool ok) {
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            tp.w[tap][0] = ok ? wv[(size_t)c0 * 27 + tap] : 0.f;
            tp.w[tap][1] = ok ? wv[(size_t)(c0 + 1) * 27 + tap] : 0.f;
        }
    }
    __device__ __forceinline__ static XT load(const char *p) { return *reinterpret_cast<const float2 *>(p); }
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static XT bload(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
        return make_float2(__uint_as_float(u.x), __uint_as_float(u.y));
    }
    __device__ __forceinline__ static void bstore(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                                  float a, float b) {
        u32x2 u;
        u.x = __float_as_uint(a);
        u.y = __float_as_uint(b);
        __builtin_amdgcn_raw_buffer_store_b64(u, r, voff, soff, 0);
    }
    __device__ __forceinline__ static XT zero() { return make_float2(0.f, 0.f); }
    __device__ __forceinline__ static void mac(const Taps &tp, int tap, XT x, float &a0, float &a1) {
        a0 = __builtin_fmaf(tp.w[tap][0], x.x, a0);
        a1 = __builtin_fmaf(tp.w[tap][1], x.y, a1);
    }
    __device__ __forceinline__ static void store(char *p, float a, float b) {
        *reinterpret_cast<float2 *>(p) = make_float2(a, b);
    }
    __device__ __forceinline__ static float lo(XT x) { return x.x; }
    __device__ __forceinline__ static float hi(XT x) { return x.y; }
    __device__ __forceinline__ static float tapw(const float *w, size_t i) { return w[i]; }
};

struct Layout {
    int n_cb[3];          // 128-channel blocks per stream
    int vis_items[3];     // B * gh * n_wrun * n_cb   (one per wave)
    int txt_items[3];     // B * n_trun * n_cb
    int vis_blocks[3], txt_blocks[3];
    int n_wrun, n_trun;
    int nblocks;
};

// Visual wave item.  Everything except the lane's channel offset is uniform.
template <typename T, int PT>
struct VisualWave {
    typedef Ops<T> O;
    __amdgpu_buffer_rsrc_t rx, ry;   // this batch's slice of the input / output stream
    int rowb;            // bytes per token row (C * sizeof(T))
    int lane_off;        // lane's channel-pair offset (bytes); the only per-lane address term
    int n_text, gt, gh, gw, h, w0;
    typename O::Taps taps;
    float acc[3][WR][2];

    // byte offset of token (t, hh, ww) inside the batch slice (< 4 GiB, checked on the host)
    __device__ __forceinline__ unsigned tok_off(int t, int hh, int ww) const {
        return (unsigned)(n_text + (t * gh + hh) * gw + ww) * (unsigned)rowb;
    }

    typename O::XT xs[2][3][WR + 2];   // double-buffered input slice (3 rows x WR+2 positions)

    // Load input slice ti (rows h-1..h+1) into buffer B; rows and positions
    // outside the grid are zero.  Every condition is wave-uniform.
    template <int B, bool EDGE>
    __device__ __forceinline__ void load_slice(int ti) {
        if (ti >= gt) return;
#pragma unroll
        for (int dh = 0; dh < 3; ++dh) {
            const int hh = h + dh - 1;
            if (hh < 0 || hh >= gh) continue;
            const unsigned row = tok_off(ti, hh, w0) - (unsigned)rowb;   // position w0 - 1
#pragma unroll
            for (int j = 0; j < WR + 2; ++j) {
                const unsigned soff = row + (unsigned)j * (unsigned)rowb;
                if (EDGE) {
                    const int ww = w0 - 1 + j;
                    xs[B][dh][j] = (ww >= 0 && ww < gw) ? O::bload(rx, lane_off, soff) : O::zero();
                } else {
                    xs[B][dh][j] = O::bload(rx, lane_off, soff);
                }
            }
        }
    }

    // Step P of the march (slice ti = 6m + P): prefetch slice ti + 1, then apply
    // slice ti.  Input slice ti contributes tap a to output slice ti + PT - a,
    // kept in accumulator slot (ti + PT - a) mod 3 == (P + PT - a) mod 3.
    template <int P, bool EDGE>
    __device__ __forceinline__ void step(int ti) {
        constexpr int CUR = P & 1;
        load_slice<CUR ^ 1, EDGE>(ti + 1);
        if (ti < gt) {
#pragma unroll
            for (int dh = 0; dh < 3; ++dh) {
                const int hh = h + dh - 1;
                if (hh < 0 || hh >= gh) continue;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const int slot = ((P + PT - a) % 3 + 3) % 3;
#pragma unroll
                    for (int e = 0; e < 3; ++e)
#pragma unroll
                        for (int j = 0; j < WR; ++j)
                            O::mac(taps, (a * 3 + dh) * 3 + e, xs[CUR][dh][j + e], acc[slot][j][0], acc[slot][j][1]);
                }
            }
        }
        constexpr int done = ((P + PT - 2) % 3 + 3) % 3;   // slot of output slice ti + PT - 2
        const int t_done = ti + PT - 2;
        if (t_done >= 0 && t_done < gt) {
            const unsigned orow = tok_off(t_done, h, w0);
#pragma unroll
            for (int j = 0; j < WR; ++j)
                if (!EDGE || w0 + j < gw)
                    O::bstore(ry, lane_off, orow + (unsigned)j * (unsigned)rowb, acc[done][j][0], acc[done][j][1]);
        }
#pragma unroll
        for (int j = 0; j < WR; ++j) acc[done][j][0] = acc[done][j][1] = 0.f;
    }

    template <bool EDGE>
    __device__ void march() {
        load_slice<0, EDGE>(0);
        // One extra empty slice (ti == gt) flushes the last output slice.
#pragma unroll 1
        for (int ti = 0; ti <= gt; ti += 6) {
            step<0, EDGE>(ti);
            if (ti + 1 > gt) break;
            step<1, EDGE>(ti + 1);
            if (ti + 2 > gt) break;
            step<2, EDGE>(ti + 2);
            if (ti + 3 > gt) break;
            step<3, EDGE>(ti + 3);
            if (ti + 4 > gt) break;
            step<4, EDGE>(ti + 4);
            if (ti + 5 > gt) break;
            step<5, EDGE>(ti + 5);
        }
    }

    __device__ void run() {
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
            for (int j = 0; j < WR; ++j) acc[s][j][0] = acc[s][j][1] = 0.f;
        if (w0 >= 1 && w0 + WR < gw)
            march<false>();
        else
            march<true>();
    }
};

template <typename T, int PT>
__device__ void visual_item(const ConvArgs &a, const Layout &L, int s, int item, int lane) {
    const int n_cb = L.n_cb[s];
    const int cb = item % n_cb;
    int rest = item / n_cb;
    const int wrun = rest % L.n_wrun;
    rest /= L.n_wrun;
    const int h = rest % a.gh;
    const int b = rest / a.gh;
    const int C = a.C[s];
    const int c0 = cb * CPW + 2 * lane;
    const bool ok = c0 < C;   // lanes past the last channel compute zeros and store nothing
    VisualWave<T, PT> wv;
    wv.rowb = C * (int)sizeof(T);
    const size_t bbytes = (size_t)a.T * wv.rowb;   // < 4 GiB, checked on the host
    wv.rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.x[s])) + (size_t)b * bbytes, 0, (int)(unsigned)bbytes,
        kBufferWord3);
    wv.ry = __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(a.y[s]) + (size_t)b * bbytes, 0,
                                              (int)(unsigned)bbytes, kBufferWord3);
    wv.lane_off = (ok ? c0 : 0) * (int)sizeof(T);
    wv.n_text = a.n_text;
    wv.gt = a.gt;
    wv.gh = a.gh;
    wv.gw = a.gw;
    wv.h = h;
    wv.w0 = wrun * WR;
    Ops<T>::load_taps(wv.taps, static_cast<const T *>(a.wv[s]), ok ? c0 : 0, ok);
    if (ok) wv.run();
}

template <typename T>
__device__ void text_item(const ConvArgs &a, const Layout &L, int s, int item, int lane) {
    typedef Ops<T> O;
    const int n_cb = L.n_cb[s];
    const int cb = item % n_cb;
    const int rest = item / n_cb;
    const int trun = rest % L.n_trun;
    const int b = rest / L.n_trun;
    const int C = a.C[s];
    const int c0 = cb * CPW + 2 * lane;
    if (c0 >= C) return;
    const int rowb = C * (int)sizeof(T);
    const char *x = static_cast<const char *>(a.x[s]) + (size_t)b * a.T * rowb + c0 * sizeof(T);
    char *y = static_cast<char *>(a.y[s]) + (size_t)b * a.T * rowb + c0 * sizeof(T);
    const T *wt = static_cast<const T *>(a.wt[s]);
    float w[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j][0] = O::tapw(wt, (size_t)c0 * 4 + j);
        w[j][1] = O::tapw(wt, (size_t)(c0 + 1) * 4 + j);
    }
    const int i0 = trun * TR;
    float xin[TR + 3][2];
#pragma unroll
    for (int m = 0; m < TR + 3; ++m) {
        const int src = i0 - 3 + m;
        if (src >= 0 && src < a.n_text) {
            const typename O::XT v = O::load(x + (size_t)src * rowb);
            xin[m][0] = O::lo(v);
            xin[m][1] = O::hi(v);
        } else {
            xin[m][0] = xin[m][1] = 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < TR; ++m) {
        const int i = i0 + m;
        if (i < a.n_text) {
            float o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o0 = __builtin_fmaf(w[j][0], xin[m + j][0], o0);
                o1 = __builtin_fmaf(w[j][1], xin[m + j][1], o1);
            }
            O::store(y + (size_t)i * rowb, o0, o1);
        }
    }
}

template <typename T, int PT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 2 : 3))) void conv_kernel(ConvArgs a, Layout L) {
    int blk = xcd_remap(blockIdx.x, L.nblocks);
    const int wave = uniform(threadIdx.x / LANES), lane = threadIdx.x % LANES;
    constexpr int WPB = NT / LANES;
#pragma unroll 1
    for (int s = 0; s < 3; ++s) {
        if (blk < L.vis_blocks[s]) {
            const int item = uniform(blk * WPB + wave);
            if (item < L.vis_items[s]) visual_item<T, PT>(a, L, s, item, lane);
            return;
        }
        blk -= L.vis_blocks[s];
        if (blk < L.txt_blocks[s]) {
            const int item = uniform(blk * WPB + wave);
            if (item < L.txt_items[s]) text_item<T>(a, L, s, item, lane);
            return;
        }
        blk -= L.txt_blocks[s];
    }
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, bool bf16, hipStream_t stream) {
    constexpr int WPB = NT / LANES;
    Layout L;
    L.n_wrun = (a.gw + WR - 1) / WR;
    L.n_trun = (a.n_text + TR - 1) / TR;
    const int n_vis = a.gt * a.gh * a.gw;
    L.nblocks = 0;
    for (int s = 0; s < 3; ++s) {
        L.n_cb[s] = (a.C[s] + CPW - 1) / CPW;
        L.vis_items[s] = n_vis ? a.B * a.gh * L.n_wrun * L.n_cb[s] : 0;
        L.txt_items[s] = a.B * L.n_trun * L.n_cb[s];
        L.vis_blocks[s] = (L.vis_items[s] + WPB - 1) / WPB;
        L.txt_blocks[s] = (L.txt_items[s] + WPB - 1) / WPB;
        L.nblocks += L.vis_blocks[s] + L.txt_blocks[s];
    }
    if (L.nblocks == 0) return hipSuccess;
    if (bf16) {
        if (a.causal_t)
            hipLaunchKernelGGL((conv_kernel<bf16_t, 2>), dim3(L.nblocks), dim3(NT), 0, stream, a, L);
        else
            hipLaunchKernelGGL((conv_kernel<bf16_t, 1>), dim3(L.nblocks), dim3(NT), 0, stream, a, L);
    } else {
        if (a.causal_t)
            hipLaunchKernelGGL((conv_kernel<float, 2>), dim3(L.nblocks), dim3(NT), 0, stream, a, L);
        else
            hipLaunchKernelGGL((conv_kernel<float, 1>), dim3(L.nblocks), dim3(NT), 0, stream, a, L);
    }
    return hipGetLastError();
}

}  // namespace kdaconv
