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
//   * conv_dw_visual_kernel: the visual tap gradients.  A block of one wave per tile row
//     walks tiles of 8 rows (4 in fp32) x 8 w positions x 128 channels (those of one
//     channel block; one block per compute unit, dealt over the channel blocks) and
//     marches each over t like the forward conv:
//     each step stages one new haloed x slice (a 3-slice ring in LDS: the slices t - P,
//     t - P + 1, t - P + 2 that dy slice t meets) and dy slice t, zero outside the grid,
//     so every input is read from memory once per tile.  Wave r takes tile row r, lane l
//     channels 2l, 2l + 1; per (a, b) tap row it reads the 10 x values of its window row
//     from LDS once (the next row's reads in flight under the current row's products) and
//     uses them for the three w taps of all 8 positions; in bf16, byte permutes pair
//     neighbouring positions so that each v_dot2_f32_bf16 does two multiply-adds.  The 27 x 2
//     running sums run on across the block's tiles, are added over the waves in LDS and
//     then into the (zeroed) weight gradients with one fp32 atomic per (channel, tap) and
//     block, in the gradients' address order so that a wave's atomics share cache lines
//     (one atomic per tile and lane-scattered addresses cost more than the march itself:
//     3.1 M atomics per stream at the 5 s video, and 113 M at a 4096 x 4096 image).
//   * conv_dw_text_kernel: the text tap gradients: about one block per compute unit, each
//     over 256 channels (4 per lane) and a share of the text tokens, 4 x 4 running sums per
//     lane, summed over the block's waves in LDS and then added with one fp32 atomic per
//     (channel, tap).
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
constexpr int kDwTokens = 2;       // text tokens per wave and token range
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

// Text tap gradients.  A block owns 256 channels (4 per lane) and walks ranges of
// kDwWaves * kDwTokens text tokens (kDwTokens per wave) with a grid stride, keeping 4 x 4
// running sums per lane; at the end the waves add their sums in LDS and the block adds each
// (channel, tap) total to the zeroed fp32 gradient with one global atomic.  The blocks of a
// channel block are the ones congruent mod the number of channel blocks.
template <typename T>
__global__ __launch_bounds__(64 * kDwWaves) void conv_dw_text_kernel(ConvBwdArgs a, int s) {
    __shared__ float red[4][4][64];   // [tap][channel of the lane's 4][lane]
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, nt = a.n_text;
    const int C = a.C[s], ncb = (C + 255) / 256, span = kDwWaves * kDwTokens, nrange = (nt + span - 1) / span;
    const int cb = blockIdx.x % ncb, c = cb * 256 + 4 * lane;
    for (int e = threadIdx.x; e < 4 * 4 * 64; e += 64 * kDwWaves) (&red[0][0][0])[e] = 0.f;
    __syncthreads();
    if (c < C) {
        // every load is issued unconditionally (a tap before the first token reads token 0
        // and contributes zero), so a token's loads are in flight together
        float st4[4][4] = {};
        for (int r = blockIdx.x / ncb; r < a.B * nrange; r += gridDim.x / ncb) {
            const int b = r / nrange, i0 = (r % nrange) * span + wave * kDwTokens, i1 = min(nt, i0 + kDwTokens);
            const T *x = static_cast<const T *>(a.x[s]) + (size_t)b * a.T * C + c;
            const T *dy = static_cast<const T *>(a.dy[s]) + (size_t)b * a.T * C + c;
            for (int i = i0; i < i1; ++i) {
                float g[4];
                ld4c(dy + (size_t)i * C, g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int src = i - 3 + j;
                    float xv[4];
                    ld4c(x + (size_t)max(src, 0) * C, xv);
#pragma unroll
                    for (int u = 0; u < 4; ++u) st4[j][u] += g[u] * (src >= 0 ? xv[u] : 0.f);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (st4[j][u] != 0.f) atomicAdd(&red[j][u][lane], st4[j][u]);
    }
    __syncthreads();
    // in the gradient's address order ([channel][4]): a wave's atomics cover one 1 KB run
    for (int e = threadIdx.x; e < 4 * 4 * 64; e += 64 * kDwWaves) {
        const int k = e % 4, cl = e / 4, u = cl % 4, l = cl / 4, ch = cb * 256 + cl;
        const float v = red[k][u][l];
        if (ch < C && v != 0.f) atomicAdd(a.dwt[s] + (size_t)ch * 4 + k, v);
    }
}

constexpr int kGW = 8;     // w positions per visual tap-gradient tile
constexpr int kGC = 128;   // channels per tile (two per lane)
// rows per tile, one wave each: 8 in bf16, 4 in fp32 (whose x ring would not fit LDS at 8)
template <typename T> struct DwTile {
    static constexpr int GH = sizeof(T) == 2 ? 8 : 4;
};

constexpr int kGX = kGW + 2;   // positions of a window row (w halo)

// The products of one window row: acc[te][ch] += sum_j dy[j][ch] x[j + te][ch] for the
// kGW positions j of a tile row and the three w taps te, on lane l's two channels.
template <typename T> struct DwOps;
template <> struct DwOps<bf16_t> {
    typedef uint32_t Raw;   // one position's channel pair (2l, 2l + 1), as stored
    // dy as bf16 pairs along w: (dy[2k][ch], dy[2k + 1][ch]) for channel ch = lo, hi
    struct Dy {
        uint32_t lo[kGW / 2], hi[kGW / 2];
    };
    __device__ __forceinline__ static Raw read(const char *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ __forceinline__ static void make_dy(const Raw (&d)[kGW], Dy &o) {
#pragma unroll
        for (int k = 0; k < kGW / 2; ++k) {
            o.lo[k] = __builtin_amdgcn_perm(d[2 * k + 1], d[2 * k], 0x05040100u);
            o.hi[k] = __builtin_amdgcn_perm(d[2 * k + 1], d[2 * k], 0x07060302u);
        }
    }
    __device__ __forceinline__ static float dot2(uint32_t x, uint32_t w, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, w), acc,
                                               false);
    }
    // byte permutes pair neighbouring positions of one channel, so each dot2 does the
    // multiply-adds of two positions
    __device__ __forceinline__ static void row(const Raw (&x)[kGX], const Dy &dy, float (*acc)[2]) {
        uint32_t plo[kGX - 1], phi[kGX - 1];   // (x[k][ch], x[k + 1][ch])
#pragma unroll
        for (int k = 0; k < kGX - 1; ++k) {
            plo[k] = __builtin_amdgcn_perm(x[k + 1], x[k], 0x05040100u);
            phi[k] = __builtin_amdgcn_perm(x[k + 1], x[k], 0x07060302u);
        }
#pragma unroll
        for (int te = 0; te < 3; ++te)
#pragma unroll
            for (int k = 0; k < kGW / 2; ++k) {
                acc[te][0] = dot2(dy.lo[k], plo[2 * k + te], acc[te][0]);
                acc[te][1] = dot2(dy.hi[k], phi[2 * k + te], acc[te][1]);
            }
    }
};
template <> struct DwOps<float> {
    typedef float2 Raw;
    struct Dy {
        float2 v[kGW];
    };
    __device__ __forceinline__ static Raw read(const char *p) { return *reinterpret_cast<const float2 *>(p); }
    __device__ __forceinline__ static void make_dy(const Raw (&d)[kGW], Dy &o) {
#pragma unroll
        for (int j = 0; j < kGW; ++j) o.v[j] = d[j];
    }
    __device__ __forceinline__ static void row(const Raw (&x)[kGX], const Dy &dy, float (*acc)[2]) {
#pragma unroll
        for (int te = 0; te < 3; ++te)
#pragma unroll
            for (int j = 0; j < kGW; ++j) {
                acc[te][0] = fmaf(dy.v[j].x, x[j + te].x, acc[te][0]);
                acc[te][1] = fmaf(dy.v[j].y, x[j + te].y, acc[te][1]);
            }
    }
};

// dW[c][a][b][e] += sum over visual positions p = (t, h, w) of dy[p][c] x[t + a - P][h + b - 1][w + e - 1][c]
// for one tile of kGH rows x kGW positions x kGC channels, marching over t.
template <typename T>
__global__ __launch_bounds__(64 * DwTile<T>::GH) void conv_dw_visual_kernel(ConvBwdArgs a, int s) {
    constexpr int ES = sizeof(T);
    constexpr int kGH = DwTile<T>::GH, NT = 64 * kGH;   // rows per tile, one wave each; threads
    constexpr int XR = kGH + 2, XC = kGX;       // haloed x tile
    constexpr int ROWB = kGC * ES;              // bytes of one position's channels
    constexpr int NCH = ROWB / 16;              // 16-byte pieces per position
    constexpr int SLOT = XR * XC * ROWB;
    constexpr int XPIECES = XR * XC * NCH, DPIECES = kGH * kGW * NCH;
    constexpr int XIT = (XPIECES + NT - 1) / NT, DIT = (DPIECES + NT - 1) / NT;
    static_assert(27 * kGC * 4 <= 3 * SLOT, "the reduction fits the x ring");
    __shared__ __attribute__((aligned(16))) char xs[3 * SLOT];          // x slices, ring by slice index mod 3
    __shared__ __attribute__((aligned(16))) char ds[kGH * kGW * ROWB];  // dy slice t

    const int C = a.C[s], gt = a.gt, gh = a.gh, gw = a.gw;
    const int nwr = (gw + kGW - 1) / kGW, nrg = (gh + kGH - 1) / kGH, ncb = (C + kGC - 1) / kGC;
    const int ntile = nwr * nrg, per = gridDim.x / (a.B * ncb);   // tiles and workgroups per (batch, channel block)
    // consecutive logical blocks (the workgroups of one channel block) on one XCD, so the
    // halo positions of neighbouring tiles come from its L2
    int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int j0 = blk % per;
    blk /= per;
    const int cb = blk % ncb, b = blk / ncb;
    const int c0 = cb * kGC;
    const int nch = (min(kGC, C - c0) * ES) / 16;   // valid pieces per position (C is a multiple of 8)
    const int P = a.causal_t ? 2 : 1;
    const int tid = threadIdx.x, r = tid >> 6, l = tid & 63;
    const char *xg = static_cast<const char *>(a.x[s]) + ((size_t)b * a.T + a.n_text) * C * ES + (size_t)c0 * ES;
    const char *dg = static_cast<const char *>(a.dy[s]) + ((size_t)b * a.T + a.n_text) * C * ES + (size_t)c0 * ES;
    int w0 = 0, h0 = 0;   // the current tile
    auto slot_of = [](int sl) { return ((sl % 3) + 3) % 3; };
    // The loads of a step's x slice sl (zeros outside the grid or outside [0, gt)) and dy
    // slice t go into registers one step ahead, so they fly under the previous step's
    // products; the stores to LDS follow that step's closing barrier.
    uint4 vx[XIT], vd[DIT];
    auto load_x = [&](int sl) {
#pragma unroll
        for (int i = 0; i < XIT; ++i) {
            const int e = tid + NT * i, pos = e / NCH, pc = e % NCH;
            const int h = h0 + pos / XC - 1, w = w0 + pos % XC - 1;
            const bool ok = e < XPIECES && pc < nch && sl >= 0 && sl < gt && h >= 0 && h < gh && w >= 0 && w < gw;
            vx[i] = ok ? *reinterpret_cast<const uint4 *>(xg + ((size_t)(sl * gh + h) * gw + w) * C * ES + 16 * pc)
                       : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&](int sl) {
        char *d = xs + slot_of(sl) * SLOT;
#pragma unroll
        for (int i = 0; i < XIT; ++i) {
            const int e = tid + NT * i;
            if (e < XPIECES) *reinterpret_cast<uint4 *>(d + (e / NCH) * ROWB + 16 * (e % NCH)) = vx[i];
        }
    };
    auto load_dy = [&](int t) {
#pragma unroll
        for (int i = 0; i < DIT; ++i) {
            const int e = tid + NT * i, pos = e / NCH, pc = e % NCH;
            const int h = h0 + pos / kGW, w = w0 + pos % kGW;
            const bool ok = t < gt && e < DPIECES && pc < nch && h < gh && w < gw;
            vd[i] = ok ? *reinterpret_cast<const uint4 *>(dg + ((size_t)(t * gh + h) * gw + w) * C * ES + 16 * pc)
                       : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_dy = [&]() {
#pragma unroll
        for (int i = 0; i < DIT; ++i) {
            const int e = tid + NT * i;
            if (e < DPIECES) *reinterpret_cast<uint4 *>(ds + (e / NCH) * ROWB + 16 * (e % NCH)) = vd[i];
        }
    };

    float acc[27][2];
#pragma unroll
    for (int k = 0; k < 27; ++k) acc[k][0] = acc[k][1] = 0.f;
    // the workgroup's tiles of its channel block, each marched over t; the sums run on
    // across them (the previous tile's last step ended with every wave done with LDS)
#pragma unroll 1
    for (int tile = j0; tile < ntile; tile += per) {
        w0 = (tile % nwr) * kGW;
        h0 = (tile / nwr) * kGH;
        load_x(-P);
        store_x(-P);
        load_x(1 - P);
        store_x(1 - P);
        load_x(2 - P);
        load_dy(0);
    #pragma unroll 1
        for (int t = 0; t < gt; ++t) {
            store_x(t - P + 2);   // its slot last held slice t - P - 1, which no wave reads any more
            store_dy();
            lds_barrier();        // LDS only: the next step's loads below stay in flight
            load_x(t - P + 3);    // the next step's (past the last step: zeros, unused)
            load_dy(t + 1);
            using Ops = DwOps<T>;
            typename Ops::Raw d[kGW], xr[2][kGX];
#pragma unroll
            for (int j = 0; j < kGW; ++j) d[j] = Ops::read(ds + (r * kGW + j) * ROWB + 2 * ES * l);
            // window row i = (ta, tb): row r + tb of slice t - P + ta; the next row's LDS
            // reads are issued before the current row's products
            auto read_row = [&](int i, typename Ops::Raw(&x)[kGX]) {
                const char *src = xs + slot_of(t - P + i / 3) * SLOT + (r + i % 3) * XC * ROWB + 2 * ES * l;
#pragma unroll
                for (int c = 0; c < kGX; ++c) x[c] = Ops::read(src + c * ROWB);
            };
            read_row(0, xr[0]);
            typename Ops::Dy dyp;
            Ops::make_dy(d, dyp);
#pragma unroll
            for (int i = 0; i < 9; ++i) {
                if (i + 1 < 9) read_row(i + 1, xr[(i + 1) & 1]);
                Ops::row(xr[i & 1], dyp, &acc[3 * i]);
            }
            lds_barrier();     // every wave is done with dy slice t and x slice t - P
        }
    }
    // the four waves' sums, added in LDS (the x ring as [27][kGC] fp32), then one atomic
    // per (channel, tap) into the zeroed gradient
    float *red = reinterpret_cast<float *>(xs);
    for (int e = tid; e < 27 * kGC; e += NT) red[e] = 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 27; ++k) {
        atomicAdd(&red[k * kGC + 2 * l], acc[k][0]);
        atomicAdd(&red[k * kGC + 2 * l + 1], acc[k][1]);
    }
    __syncthreads();
    // in the gradient's address order ([channel][27]), so a wave's atomics cover two
    // consecutive cache lines instead of one line per lane
    for (int e = tid; e < 27 * kGC; e += NT) {
        const int k = e % 27, cl = e / 27, ch = c0 + cl;
        const float v = red[k * kGC + cl];
        if (ch < C && v != 0.f) atomicAdd(a.dwv[s] + (size_t)c0 * 27 + e, v);
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
        if (a.n_text > 0) {
            // text taps: one block per compute unit (a multiple of the channel-block count),
            // at most one per token range
            const int ncb = (a.C[s] + 255) / 256;
            const int nrange = (a.n_text + kDwWaves * kDwTokens - 1) / (kDwWaves * kDwTokens);
            const int per_cb = std::max(1, std::min(a.B * nrange, kCUs / ncb));
            hipLaunchKernelGGL((conv_dw_text_kernel<T>), dim3(ncb * per_cb), dim3(64 * kDwWaves), 0, stream, a, s);
        }
        if (vis) {
            // about as many workgroups as fit the chip at once (one per compute unit by their
            // LDS), dealt over the (batch, channel block) pairs
            constexpr int gh = DwTile<T>::GH;
            const int nwr = (a.gw + kGW - 1) / kGW, nrg = (a.gh + gh - 1) / gh, ncb = (a.C[s] + kGC - 1) / kGC;
            const int per = std::max(1, std::min(nwr * nrg, kCUs / (a.B * ncb)));
            hipLaunchKernelGGL((conv_dw_visual_kernel<T>), dim3(a.B * ncb * per), dim3(64 * gh), 0, stream, a, s);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_backward(const ConvBwdArgs &a, bool bf16, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace kdaconv
