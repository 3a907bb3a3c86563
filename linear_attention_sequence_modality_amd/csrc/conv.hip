// Modality-aware depthwise short convolution (gfx950).
//
// Chimera pages: the conv runs before every KDA update, separately per
// modality -- a causal 1D depthwise conv over text tokens and a depthwise 3D
// conv over the visual tokens on their (t, h, w) grid (rainbus "core method";
// genai-atlas "How it works").  Taps: text 4 (last tap on the current token),
// visual 3x3x3 with zero padding; time offset P = 1 (symmetric) or 2 (causal).
//
// Design (HBM/VALU bound, no matrix cores: a depthwise conv has no channel
// contraction):
//   * one thread owns CG adjacent channels of one stream and a run of WR
//     consecutive w positions of one (b, h) row, and marches over t.  Each
//     input slice t is loaded once (3 rows x (WR+2) positions) and feeds the
//     three output slices t-1, t, t+1 from registers: a 3-deep accumulator
//     ring whose slot index is static after unrolling the march by 3;
//   * lanes of a wave take consecutive channel pairs, so each wave load is a
//     contiguous 256 B (bf16) / 512 B (fp32) slice of one token row;
//   * blocks are remapped so each XCD works on a contiguous range of rows,
//     keeping the h-1/h/h+1 halo rows in that XCD's L2;
//   * text tokens are a separate block range: a thread slides a 4-tap window
//     over TR consecutive text tokens.
#include "common.h"
#include "launch.h"

namespace kdaconv {
namespace {

constexpr int CG = 2;     // channels per thread
constexpr int WR = 8;     // w positions per thread
constexpr int TR = 8;     // text tokens per thread
constexpr int NT = 256;   // threads per block

template <typename T> struct Vec2;
template <> struct Vec2<bf16_t> {
    __device__ __forceinline__ static void load(const bf16_t *p, float (&o)[2]) {
        uint32_t u = *reinterpret_cast<const uint32_t *>(p);
        o[0] = bf16_lo(u);
        o[1] = bf16_hi(u);
    }
    __device__ __forceinline__ static void store(bf16_t *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
};
template <> struct Vec2<float> {
    __device__ __forceinline__ static void load(const float *p, float (&o)[2]) {
        float2 u = *reinterpret_cast<const float2 *>(p);
        o[0] = u.x;
        o[1] = u.y;
    }
    __device__ __forceinline__ static void store(float *p, float a, float b) {
        *reinterpret_cast<float2 *>(p) = make_float2(a, b);
    }
};

struct Layout {
    int n_cg[3];          // channel groups per stream
    int vis_items[3];     // B * gh * n_wrun * n_cg
    int txt_items[3];     // B * n_trun * n_cg
    int vis_blocks[3], txt_blocks[3];
    int n_wrun, n_trun;
    int nblocks;
};

template <typename T, int PT>
struct VisualThread {
    const T *x;
    T *y;
    int C, T_len, n_text, gt, gh, gw, h, w0;
    float wv[27][CG];
    float acc[3][WR][CG];

    // Input slice ti contributes tap a to output slice ti + PT - a, which
    // lives in accumulator slot (ti + PT - a) mod 3 == (P + PT - a) mod 3.
    template <int P>
    __device__ __forceinline__ void step(int ti) {
        const bool t_ok = ti < gt;
#pragma unroll
        for (int dh = 0; dh < 3; ++dh) {
            const int hh = h + dh - 1;
            const bool row_ok = t_ok && hh >= 0 && hh < gh;
            float xin[WR + 2][CG];
            const size_t row_tok = (size_t)n_text + ((size_t)ti * gh + hh) * gw;
#pragma unroll
            for (int j = 0; j < WR + 2; ++j) {
                const int ww = w0 - 1 + j;
                if (row_ok && ww >= 0 && ww < gw) {
                    Vec2<T>::load(x + (row_tok + ww) * C, xin[j]);
                } else {
#pragma unroll
                    for (int c = 0; c < CG; ++c) xin[j][c] = 0.f;
                }
            }
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                constexpr int dummy = 0;
                (void)dummy;
                const int slot = ((P + PT - a) % 3 + 3) % 3;
#pragma unroll
                for (int e = 0; e < 3; ++e) {
#pragma unroll
                    for (int j = 0; j < WR; ++j) {
#pragma unroll
                        for (int c = 0; c < CG; ++c)
                            acc[slot][j][c] = __builtin_fmaf(wv[(a * 3 + dh) * 3 + e][c],
                                                             xin[j + e][c], acc[slot][j][c]);
                    }
                }
            }
        }
        // Output slice ti + PT - 2 has now received all its taps.
        constexpr int done = ((P + PT - 2) % 3 + 3) % 3;
        const int t_done = ti + PT - 2;
        if (t_done >= 0 && t_done < gt) {
            const size_t row_tok = (size_t)n_text + ((size_t)t_done * gh + h) * gw;
#pragma unroll
            for (int j = 0; j < WR; ++j)
                if (w0 + j < gw) Vec2<T>::store(y + (row_tok + w0 + j) * C, acc[done][j][0],
                                                acc[done][j][1]);
        }
#pragma unroll
        for (int j = 0; j < WR; ++j)
#pragma unroll
            for (int c = 0; c < CG; ++c) acc[done][j][c] = 0.f;
    }

    __device__ void run() {
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
            for (int j = 0; j < WR; ++j)
#pragma unroll
                for (int c = 0; c < CG; ++c) acc[s][j][c] = 0.f;
        // One extra all-zero slice (ti == gt) flushes the last output slice.
        for (int ti = 0; ti <= gt; ti += 3) {
            step<0>(ti);
            if (ti + 1 > gt) break;
            step<1>(ti + 1);
            if (ti + 2 > gt) break;
            step<2>(ti + 2);
        }
    }
};

template <typename T>
__device__ void visual_item(const ConvArgs &a, const Layout &L, int s, int item) {
    const int n_cg = L.n_cg[s];
    const int cg = item % n_cg;
    int rest = item / n_cg;
    const int wrun = rest % L.n_wrun;
    rest /= L.n_wrun;
    const int h = rest % a.gh;
    const int b = rest / a.gh;
    const int C = a.C[s];
    const int c0 = cg * CG;

    const T *wv = static_cast<const T *>(a.wv[s]);
    const size_t boff = (size_t)b * a.T * C + c0;
    if (a.causal_t) {
        VisualThread<T, 2> th;
        th.x = static_cast<const T *>(a.x[s]) + boff;
        th.y = static_cast<T *>(a.y[s]) + boff;
        th.C = C; th.T_len = a.T; th.n_text = a.n_text;
        th.gt = a.gt; th.gh = a.gh; th.gw = a.gw; th.h = h; th.w0 = wrun * WR;
#pragma unroll
        for (int tap = 0; tap < 27; ++tap)
#pragma unroll
            for (int c = 0; c < CG; ++c)
                th.wv[tap][c] = ElemIO<T>::load(wv + (size_t)(c0 + c) * 27 + tap);
        th.run();
    } else {
        VisualThread<T, 1> th;
        th.x = static_cast<const T *>(a.x[s]) + boff;
        th.y = static_cast<T *>(a.y[s]) + boff;
        th.C = C; th.T_len = a.T; th.n_text = a.n_text;
        th.gt = a.gt; th.gh = a.gh; th.gw = a.gw; th.h = h; th.w0 = wrun * WR;
#pragma unroll
        for (int tap = 0; tap < 27; ++tap)
#pragma unroll
            for (int c = 0; c < CG; ++c)
                th.wv[tap][c] = ElemIO<T>::load(wv + (size_t)(c0 + c) * 27 + tap);
        th.run();
    }
}

template <typename T>
__device__ void text_item(const ConvArgs &a, const Layout &L, int s, int item) {
    const int n_cg = L.n_cg[s];
    const int cg = item % n_cg;
    const int rest = item / n_cg;
    const int trun = rest % L.n_trun;
    const int b = rest / L.n_trun;
    const int C = a.C[s];
    const int c0 = cg * CG;
    const T *x = static_cast<const T *>(a.x[s]) + (size_t)b * a.T * C + c0;
    T *y = static_cast<T *>(a.y[s]) + (size_t)b * a.T * C + c0;
    const T *wt = static_cast<const T *>(a.wt[s]);
    float w[4][CG];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < CG; ++c) w[j][c] = ElemIO<T>::load(wt + (size_t)(c0 + c) * 4 + j);
    const int i0 = trun * TR;
    float xin[TR + 3][CG];
#pragma unroll
    for (int m = 0; m < TR + 3; ++m) {
        const int src = i0 - 3 + m;
        if (src >= 0 && src < a.n_text) {
            Vec2<T>::load(x + (size_t)src * C, xin[m]);
        } else {
#pragma unroll
            for (int c = 0; c < CG; ++c) xin[m][c] = 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < TR; ++m) {
        const int i = i0 + m;
        if (i < a.n_text) {
            float o[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(w[j][c], xin[m + j][c], acc);
                o[c] = acc;
            }
            Vec2<T>::store(y + (size_t)i * C, o[0], o[1]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(NT) void conv_kernel(ConvArgs a, Layout L) {
    int blk = xcd_remap(blockIdx.x, L.nblocks);
#pragma unroll 1
    for (int s = 0; s < 3; ++s) {
        if (blk < L.vis_blocks[s]) {
            const int item = blk * NT + threadIdx.x;
            if (item < L.vis_items[s]) visual_item<T>(a, L, s, item);
            return;
        }
        blk -= L.vis_blocks[s];
        if (blk < L.txt_blocks[s]) {
            const int item = blk * NT + threadIdx.x;
            if (item < L.txt_items[s]) text_item<T>(a, L, s, item);
            return;
        }
        blk -= L.txt_blocks[s];
    }
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, bool bf16, hipStream_t stream) {
    Layout L;
    L.n_wrun = (a.gw + WR - 1) / WR;
    L.n_trun = (a.n_text + TR - 1) / TR;
    const int n_vis = a.gt * a.gh * a.gw;
    L.nblocks = 0;
    for (int s = 0; s < 3; ++s) {
        L.n_cg[s] = a.C[s] / CG;
        L.vis_items[s] = n_vis ? a.B * a.gh * L.n_wrun * L.n_cg[s] : 0;
        L.txt_items[s] = a.B * L.n_trun * L.n_cg[s];
        L.vis_blocks[s] = (L.vis_items[s] + NT - 1) / NT;
        L.txt_blocks[s] = (L.txt_items[s] + NT - 1) / NT;
        L.nblocks += L.vis_blocks[s] + L.txt_blocks[s];
    }
    if (L.nblocks == 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(conv_kernel<bf16_t>, dim3(L.nblocks), dim3(NT), 0, stream, a, L);
    else
        hipLaunchKernelGGL(conv_kernel<float>, dim3(L.nblocks), dim3(NT), 0, stream, a, L);
    return hipGetLastError();
}

}  // namespace kdaconv
