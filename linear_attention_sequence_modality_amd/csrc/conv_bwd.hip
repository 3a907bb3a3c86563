// Backward of the modality-aware depthwise short conv.
//
// The forward sums tap * input over a fixed neighbourhood, so each input
// receives tap * dy of every output it feeds (the conv with mirrored
// offsets), and each tap the sum of input * dy over the outputs:
//   text  (y_i = sum_j w_j x_{i-3+j}):  dx_i = sum_j w_j dy_{i+3-j},   dw_j = sum_i dy_i x_{i-3+j}
//   visual (y_p = sum_o W_o x_{p+o}):   dx_p = sum_o W_o dy_{p-o},     dW_o = sum_p dy_p x_{p+o}
// with o = (a - P, b - 1, e - 1) over the 3x3x3 taps (P = 1 symmetric, 2 time-causal)
// and every term outside the stream's modality region dropped.
//   * conv_dx_kernel: one thread per (token, channel pair), 4 or 27 gathers of dy.
//   * conv_dw_kernel: about one block per compute unit, each over 256 channels (4 per
//     lane) and a share of the tokens, 31 x 4 running sums per lane, summed over the
//     block's waves in LDS and then added with one fp32 atomic per (channel, tap) into
//     the (zeroed) weight gradients.
//   * symmetric time padding: the visual input gradient is the forward conv kernel
//     run on dy with the taps mirrored through the centre.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace kdaconv {
namespace {

constexpr int kDxThreads = 256;
constexpr int kDwWaves = 8;        // waves per tap-gradient block
constexpr int kDwTokens = 8;       // tokens per wave and token range
constexpr int kCUs = 256;          // compute units the tap-gradient grid is sized for

__device__ __forceinline__ float ldf(const float *p) { return *p; }
__device__ __forceinline__ float ldf(const bf16_t *p) { return (float)*p; }
__device__ __forceinline__ void stf(float *p, float x) { *p = x; }
__device__ __forceinline__ void stf(bf16_t *p, float x) { *p = (bf16_t)x; }

// Stream position of visual (t, h, w), or -1 outside the grid.
__device__ __forceinline__ int vpos(const ConvBwdArgs &a, int t, int h, int w) {
    if (t < 0 || t >= a.gt || h < 0 || h >= a.gh || w < 0 || w >= a.gw) return -1;
    return a.n_text + (t * a.gh + h) * a.gw + w;
}

// Tokens [0, nt) of every batch (nt = T, or n_text when the visual part is done elsewhere).
template <typename T>
__global__ __launch_bounds__(kDxThreads) void conv_dx_kernel(ConvBwdArgs a, int s, int nt) {
    const int C = a.C[s], npair = C / 2;
    const size_t total = (size_t)a.B * nt * npair;
    const T *dy = static_cast<const T *>(a.dy[s]);
    const T *wt = static_cast<const T *>(a.wt[s]), *wv = static_cast<const T *>(a.wv[s]);
    T *dx = static_cast<T *>(a.dx[s]);
    const int P = a.causal_t ? 2 : 1;
    for (size_t e = (size_t)blockIdx.x * kDxThreads + threadIdx.x; e < total; e += (size_t)gridDim.x * kDxThreads) {
        const int c = 2 * (int)(e % npair);
        const size_t bt = e / npair;
        const int i = (int)(bt % nt);
        const size_t base = (bt / nt) * a.T * C;   // this batch's first token
        float g0 = 0.f, g1 = 0.f;
        if (i < a.n_text) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int o = i + 3 - j;
                const size_t oc = (size_t)(o < a.n_text ? o : i) * C;   // unconditional load, zero weight
                const float y0 = ldf(dy + base + oc + c), y1 = ldf(dy + base + oc + c + 1);
                g0 += ldf(wt + (size_t)c * 4 + j) * (o < a.n_text ? y0 : 0.f);
                g1 += ldf(wt + (size_t)(c + 1) * 4 + j) * (o < a.n_text ? y1 : 0.f);
            }
        } else {
            const int p = i - a.n_text, t = p / (a.gh * a.gw), hw = p % (a.gh * a.gw), h = hw / a.gw, w = hw % a.gw;
#pragma unroll
            for (int ta = 0; ta < 3; ++ta)
#pragma unroll
                for (int tb = 0; tb < 3; ++tb)
#pragma unroll
                    for (int te = 0; te < 3; ++te) {
                        const int o = vpos(a, t - (ta - P), h - (tb - 1), w - (te - 1));
                        const int tap = (ta * 3 + tb) * 3 + te;
                        const size_t oc = (size_t)(o >= 0 ? o : i) * C;   // unconditional load, zero weight
                        const float y0 = ldf(dy + base + oc + c), y1 = ldf(dy + base + oc + c + 1);
                        g0 += ldf(wv + (size_t)c * 27 + tap) * (o >= 0 ? y0 : 0.f);
                        g1 += ldf(wv + (size_t)(c + 1) * 27 + tap) * (o >= 0 ? y1 : 0.f);
                    }
        }
        stf(dx + base + (size_t)i * C + c, g0);
        stf(dx + base + (size_t)i * C + c + 1, g1);
    }
}

// 4 consecutive channels as fp32.
__device__ __forceinline__ void ld4c(const float *p, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void ld4c(const bf16_t *p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
}

// A block owns 256 channels (4 per lane) and walks token ranges of kDwWaves * kDwTokens
// tokens (one slice of kDwTokens per wave) with a grid stride, keeping 31 x 4 running sums
// per lane across all of them; at the end the waves add their sums in LDS and the block
// adds each (channel, tap) total to the zeroed fp32 gradient with one global atomic.  The
// blocks of a channel block are the ones congruent mod the number of channel blocks.
template <typename T>
__global__ __launch_bounds__(64 * kDwWaves) void conv_dw_kernel(ConvBwdArgs a, int s) {
    __shared__ float red[31][4][64];   // [tap: 4 text then 27 visual][channel of the lane's 4][lane]
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int C = a.C[s], ncb = (C + 255) / 256, span = kDwWaves * kDwTokens, nrange = (a.T + span - 1) / span;
    const int cb = blockIdx.x % ncb, c = cb * 256 + 4 * lane;
    for (int e = threadIdx.x; e < 31 * 4 * 64; e += 64 * kDwWaves) (&red[0][0][0])[e] = 0.f;
    __syncthreads();
    if (c < C) {
        const int P = a.causal_t ? 2 : 1;
        // every load is issued unconditionally (a position off the grid reads the token
        // itself and contributes zero), so a token's loads are in flight together
        float st4[4][4] = {}, sv[27][4] = {};
        for (int r = blockIdx.x / ncb; r < a.B * nrange; r += gridDim.x / ncb) {
            const int b = r / nrange, i0 = (r % nrange) * span + wave * kDwTokens, i1 = min(a.T, i0 + kDwTokens);
            const T *x = static_cast<const T *>(a.x[s]) + (size_t)b * a.T * C + c;
            const T *dy = static_cast<const T *>(a.dy[s]) + (size_t)b * a.T * C + c;
            for (int i = i0; i < i1; ++i) {
                float g[4];
                ld4c(dy + (size_t)i * C, g);
                if (i < a.n_text) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int src = i - 3 + j;
                        float xv[4];
                        ld4c(x + (size_t)max(src, 0) * C, xv);
#pragma unroll
                        for (int u = 0; u < 4; ++u) st4[j][u] += g[u] * (src >= 0 ? xv[u] : 0.f);
                    }
                } else {
                    const int p = i - a.n_text, t = p / (a.gh * a.gw), hw = p % (a.gh * a.gw), h = hw / a.gw,
                              w = hw % a.gw;
#pragma unroll
                    for (int ta = 0; ta < 3; ++ta)
#pragma unroll
                        for (int tb = 0; tb < 3; ++tb)
#pragma unroll
                            for (int te = 0; te < 3; ++te) {
                                const int src = vpos(a, t + ta - P, h + tb - 1, w + te - 1);
                                float xv[4];
                                ld4c(x + (size_t)(src >= 0 ? src : i) * C, xv);
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    sv[(ta * 3 + tb) * 3 + te][u] += g[u] * (src >= 0 ? xv[u] : 0.f);
                            }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (st4[j][u] != 0.f) atomicAdd(&red[j][u][lane], st4[j][u]);
#pragma unroll
            for (int k = 0; k < 27; ++k)
                if (sv[k][u] != 0.f) atomicAdd(&red[4 + k][u][lane], sv[k][u]);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 31 * 4 * 64; e += 64 * kDwWaves) {
        const int k = e / 256, u = (e / 64) % 4, l = e % 64, ch = cb * 256 + 4 * l + u;
        const float v = red[k][u][l];
        if (ch < C && v != 0.f) atomicAdd(k < 4 ? a.dwt[s] + (size_t)ch * 4 + k : a.dwv[s] + (size_t)ch * 27 + (k - 4), v);
    }
}

// The visual taps mirrored through the centre (tap 26 - k), in the stream dtype: the
// symmetric conv's input gradient is the forward conv of dy with these taps.
template <typename T>
__global__ void flip_taps_kernel(const T *w, T *out, int C) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < C * 27; e += gridDim.x * blockDim.x)
        out[e] = w[(e / 27) * 27 + 26 - e % 27];
}

__global__ void zero_kernel(float *p, size_t n) {
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        p[e] = 0.f;
}

template <typename T>
hipError_t launch_typed(const ConvBwdArgs &a, hipStream_t stream) {
    const bool vis = a.gt * a.gh * a.gw > 0;
    // Symmetric time padding: the visual input gradient is the forward conv of dy with
    // mirrored taps (its text outputs are redone below).  The mirrored taps are parked in
    // the visual tap-gradient buffers, which are zeroed only after that conv has read them.
    const bool mirrored = vis && !a.causal_t;
    if (mirrored) {
        ConvArgs f;
        for (int s = 0; s < 3; ++s) {
            hipLaunchKernelGGL((flip_taps_kernel<T>), dim3(64), dim3(256), 0, stream, static_cast<const T *>(a.wv[s]),
                               reinterpret_cast<T *>(a.dwv[s]), a.C[s]);
            f.x[s] = a.dy[s];
            f.y[s] = a.dx[s];
            f.wt[s] = a.wt[s];
            f.wv[s] = a.dwv[s];
            f.C[s] = a.C[s];
            f.hx[s] = nullptr;
        }
        f.B = a.B;
        f.T = a.T;
        f.n_text = a.n_text;
        f.gt = a.gt;
        f.gh = a.gh;
        f.gw = a.gw;
        f.causal_t = 0;
        f.n_hist = 0;
        hipError_t e = launch_conv(f, sizeof(T) == 2, stream);
        if (e != hipSuccess) return e;
    }
    for (int s = 0; s < 3; ++s) {
        // input gradients of the tokens the mirrored conv did not cover (all of them otherwise)
        const int nt = mirrored ? a.n_text : a.T;
        const size_t pairs = (size_t)a.B * nt * (a.C[s] / 2);
        if (pairs) {
            const size_t want = (pairs + kDxThreads - 1) / kDxThreads;
            const int gx = (int)(want < 65536 ? want : 65536);
            hipLaunchKernelGGL((conv_dx_kernel<T>), dim3(gx), dim3(kDxThreads), 0, stream, a, s, nt);
        }
        const size_t nz_t = (size_t)a.C[s] * 4, nz_v = (size_t)a.C[s] * 27;
        hipLaunchKernelGGL(zero_kernel, dim3(64), dim3(256), 0, stream, a.dwt[s], nz_t);
        hipLaunchKernelGGL(zero_kernel, dim3(64), dim3(256), 0, stream, a.dwv[s], nz_v);
        // one block per compute unit (a multiple of the channel-block count), at most one per range
        const int ncb = (a.C[s] + 255) / 256, nrange = (a.T + kDwWaves * kDwTokens - 1) / (kDwWaves * kDwTokens);
        const int per_cb = std::max(1, std::min(a.B * nrange, kCUs / ncb));
        hipLaunchKernelGGL((conv_dw_kernel<T>), dim3(ncb * per_cb), dim3(64 * kDwWaves), 0, stream, a, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_backward(const ConvBwdArgs &a, bool bf16, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace kdaconv
