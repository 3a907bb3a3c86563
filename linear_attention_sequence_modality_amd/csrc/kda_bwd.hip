// Backward pass of the KDA scan (gradients of q, k, v, alpha, beta and the
// initial state, given those of o and the final state), chunk by chunk.
//
// Per chunk of C = 64 rows r (G_r = sum_{u<=r} log alpha_u per key channel,
// gam = 2^(G log2 e), gC = G of the last row), the forward is regrouped as
//   Kt = gam K, Kd = K / gam, Qt = gam Q, Kh = exp(gC - G) K,
//   A = strict_lower(Kt Kd^T), Bq = lower(Qt Kd^T), Tm = (I + Diag(beta) A)^-1,
//   X = Diag(beta) V, Y = Diag(beta) Kt, W = Tm Y, Ut = Tm X,
//   U = Ut - W S, O = Qt S + Bq U, S' = Diag(exp(gC)) S + Kh^T U
// and its adjoint, for dO and dS' (the gradient of the state after the chunk), is
//   dU = Bq^T dO + Kh dS',  dS = Qt^T dO + Diag(exp(gC)) dS' - W^T dU,
//   dBq = lower(dO U^T), dQt = dO S^T + dBq Kd, dKh = U dS'^T, dW = -dU S^T,
//   dTm = dU X^T + dW Y^T, dM = -Tm^T dTm Tm^T, dA = strict_lower(Diag(beta) dM),
//   dX = Tm^T dU, dY = Tm^T dW, dKt = Diag(beta) dY + dA Kd, dKd = dA^T Kt + dBq^T Qt,
//   dbeta = rowsum(dM A) + rowsum(dX V) + rowsum(dY Kt), dV = Diag(beta) dX,
//   dQ = gam dQt, dK = gam dKt + dKd / gam + exp(gC - G) dKh,
//   dG = dQt Qt + dKt Kt - dKd Kd - dKh Kh  (+ on the last row: colsum(dKh Kh) + exp(gC) rowsum(dS' S)),
//   dlog alpha = reverse cumulative sum of dG over the chunk, dalpha = dlog alpha / alpha.
//
// Four launches, all fp32 inside:
//   1. bwd_prep:    per (batch, head, chunk), in parallel: Qt, Kh, W, Ut, Bq, exp(gC).
//   2. bwd_states:  per (batch, head, 64 value columns), in chunk order: the state
//                   at the start of every chunk.
//   3. bwd_reverse: per (batch, head, 64 value columns), in reverse chunk order:
//                   dS' of every chunk and the gradient of the initial state.
//   4. bwd_intra:   per (batch, head, chunk), in parallel: the gradients of the
//                   chunk's tokens.
// The dense products run through one LDS-tiled fp32 routine (64 x 64 output
// tiles, 4 x 4 per thread); this pass is written for exactness first.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "launch.h"

namespace kdaconv {
namespace {

constexpr int BC = kChunk;      // rows per chunk
constexpr int BT = 256;         // threads per workgroup
constexpr int VS = 64;          // value columns per workgroup of the two ordered passes

// ---- small dense helpers (all threads of the workgroup take part) ------------

enum Mask { kNoMask = 0, kLower = 1, kStrictLower = 2 };

// C[m][n] = scale * sum_k op(A)[m][k] op(B)[k][n]  (+ C when acc), for m < M, n < N;
// op(A)[m][k] = TA ? A[k*lda + m] : A[m*lda + k]; op(B)[k][n] = TB ? B[n*ldb + k] : B[k*ldb + n].
// M, N multiples of 64, K a multiple of 16.  The mask zeroes the result above
// the diagonal (kLower) or on and above it (kStrictLower).  Ends with a barrier.
template <bool TA, bool TB>
__device__ void gemm(float *C, int ldc, const float *A, int lda, const float *B, int ldb, int M, int N, int K,
                     float scale, bool acc, Mask mask, float (*tA)[65], float (*tB)[65]) {
    const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;   // this thread: rows 4tr.., cols 4tc..
    for (int m0 = 0; m0 < M; m0 += 64)
        for (int n0 = 0; n0 < N; n0 += 64) {
            float c[4][4] = {};
            for (int k0 = 0; k0 < K; k0 += 16) {
                // tA[k][m] and tB[k][n] for 16 k and 64 m / n
                for (int e = tid; e < 16 * 64; e += BT) {
                    const int kk = e / 64, mm = e % 64;
                    tA[kk][mm] = TA ? A[(size_t)(k0 + kk) * lda + m0 + mm] : A[(size_t)(m0 + mm) * lda + k0 + kk];
                    tB[kk][mm] = TB ? B[(size_t)(n0 + mm) * ldb + k0 + kk] : B[(size_t)(k0 + kk) * ldb + n0 + mm];
                }
                __syncthreads();
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    float a[4], b[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[i] = tA[kk][4 * tr + i];
                        b[i] = tB[kk][4 * tc + i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) c[i][j] = fmaf(a[i], b[j], c[i][j]);
                }
                __syncthreads();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = m0 + 4 * tr + i, n = n0 + 4 * tc + j;
                    float x = scale * c[i][j];
                    if ((mask == kLower && n > m) || (mask == kStrictLower && n >= m)) x = 0.f;
                    float *p = C + (size_t)m * ldc + n;
                    *p = acc ? *p + x : x;
                }
        }
    __syncthreads();
}

__device__ __forceinline__ float ld(const float *p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t *p) { return (float)*p; }
__device__ __forceinline__ void st(float *p, float x) { *p = x; }
__device__ __forceinline__ void st(bf16_t *p, float x) { *p = (bf16_t)x; }

// Per-chunk matrices rebuilt from the inputs (fp32, row-major, in the
// workgroup's scratch): the chunk's rows past the stream's end are zero.
struct ChunkMats {
    float *Q, *K, *V, *G, *Kt, *Kd, *Qt, *Kh, *A, *Bq, *Tm, *X, *Y, *W, *Ut;
    float *beta, *eC;   // [BC], [DK]
};

template <typename T>
__device__ void chunk_forward(const KdaBwdArgs &a, const ChunkMats &c, int bh, int n, float (*tA)[65],
                              float (*tB)[65]) {
    const int DK = a.dk, DV = a.dv, H = a.H, tid = threadIdx.x;
    const int b = bh / H, h = bh % H, t0 = n * BC, nr = min(BC, a.T - t0);
    const T *q = static_cast<const T *>(a.q), *k = static_cast<const T *>(a.k), *v = static_cast<const T *>(a.v);
    const T *al = static_cast<const T *>(a.alpha), *be = static_cast<const T *>(a.beta);
    auto tok = [&](int r) { return ((size_t)b * a.T + t0 + r) * H + h; };
    for (int e = tid; e < BC * DK; e += BT) {
        const int r = e / DK, ch = e % DK;
        const bool ok = r < nr;
        c.Q[e] = ok ? ld(q + tok(r) * DK + ch) : 0.f;
        c.K[e] = ok ? ld(k + tok(r) * DK + ch) : 0.f;
    }
    for (int e = tid; e < BC * DV; e += BT) {
        const int r = e / DV, ch = e % DV;
        c.V[e] = r < nr ? ld(v + tok(r) * DV + ch) : 0.f;
    }
    if (tid < BC) c.beta[tid] = tid < nr ? ld(be + tok(tid)) : 0.f;
    // G: cumulative sum of log alpha down the rows (rows past the end add 0)
    for (int ch = tid; ch < DK; ch += BT) {
        float g = 0.f;
        for (int r = 0; r < BC; ++r) {
            if (r < nr) g += logf(ld(al + tok(r) * DK + ch));
            c.G[r * DK + ch] = g;
        }
        c.eC[ch] = expf(g);
    }
    __syncthreads();
    for (int e = tid; e < BC * DK; e += BT) {
        const int ch = e % DK;
        const float g = c.G[e], gc = logf(c.eC[ch]);
        const float gm = expf(g), kk = c.K[e];
        c.Kt[e] = gm * kk;
        c.Kd[e] = kk / gm;
        c.Qt[e] = gm * c.Q[e];
        c.Kh[e] = expf(gc - g) * kk;
    }
    __syncthreads();
    gemm<false, true>(c.A, BC, c.Kt, DK, c.Kd, DK, BC, BC, DK, 1.f, false, kStrictLower, tA, tB);
    gemm<false, true>(c.Bq, BC, c.Qt, DK, c.Kd, DK, BC, BC, DK, 1.f, false, kLower, tA, tB);
    // Tm = (I + Diag(beta) A)^-1 (unit lower triangular): column j by forward substitution
    if (tid < BC) {
        const int j = tid;
        for (int i = 0; i < BC; ++i) {
            float x = i == j ? 1.f : 0.f;
            if (i > j) {
                float s = 0.f;
                for (int u = j; u < i; ++u) s += c.A[i * BC + u] * c.Tm[u * BC + j];
                x = -c.beta[i] * s;
            }
            c.Tm[i * BC + j] = x;
        }
    }
    for (int e = tid; e < BC * DV; e += BT) c.X[e] = c.beta[e / DV] * c.V[e];
    for (int e = tid; e < BC * DK; e += BT) c.Y[e] = c.beta[e / DK] * c.Kt[e];
    __syncthreads();
    gemm<false, false>(c.W, DK, c.Tm, BC, c.Y, DK, BC, DK, BC, 1.f, false, kNoMask, tA, tB);
    gemm<false, false>(c.Ut, DV, c.Tm, BC, c.X, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);
}

// Scratch of one workgroup: the ChunkMats plus the backward's temporaries.
__device__ ChunkMats carve(float *s, int DK, int DV, float **rest) {
    ChunkMats c;
    const size_t mk = (size_t)BC * DK, mv = (size_t)BC * DV, mc = (size_t)BC * BC;
    c.Q = s; s += mk;
    c.K = s; s += mk;
    c.V = s; s += mv;
    c.G = s; s += mk;
    c.Kt = s; s += mk;
    c.Kd = s; s += mk;
    c.Qt = s; s += mk;
    c.Kh = s; s += mk;
    c.A = s; s += mc;
    c.Bq = s; s += mc;
    c.Tm = s; s += mc;
    c.X = s; s += mv;
    c.Y = s; s += mk;
    c.W = s; s += mk;
    c.Ut = s; s += mv;
    c.beta = s; s += BC;
    c.eC = s; s += DK;
    *rest = s;
    return c;
}

// Per-chunk record written by bwd_prep and read by the two ordered passes.
struct Rec {
    float *Qt, *Kh, *W, *Ut, *Bq, *eC;
};
__device__ Rec rec_at(const KdaBwdArgs &a, int bh, int n) {
    const size_t mk = (size_t)BC * a.dk, mv = (size_t)BC * a.dv;
    float *p = a.rec + ((size_t)bh * a.n_chunks + n) * a.rec_floats;
    Rec r;
    r.Qt = p; p += mk;
    r.Kh = p; p += mk;
    r.W = p; p += mk;
    r.Ut = p; p += mv;
    r.Bq = p; p += (size_t)BC * BC;
    r.eC = p;
    return r;
}

template <typename T>
__global__ __launch_bounds__(BT) void bwd_prep_kernel(KdaBwdArgs a) {
    __shared__ float tA[16][65], tB[16][65];
    float *rest;
    const ChunkMats c = carve(a.scratch + (size_t)blockIdx.x * a.scratch_floats, a.dk, a.dv, &rest);
    const int items = a.B * a.H * a.n_chunks;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int bh = it / a.n_chunks, n = it % a.n_chunks;
        chunk_forward<T>(a, c, bh, n, tA, tB);
        const Rec r = rec_at(a, bh, n);
        const int DK = a.dk, DV = a.dv;
        for (int e = threadIdx.x; e < BC * DK; e += BT) {
            r.Qt[e] = c.Qt[e];
            r.Kh[e] = c.Kh[e];
            r.W[e] = c.W[e];
        }
        for (int e = threadIdx.x; e < BC * DV; e += BT) r.Ut[e] = c.Ut[e];
        for (int e = threadIdx.x; e < BC * BC; e += BT) r.Bq[e] = c.Bq[e];
        for (int e = threadIdx.x; e < DK; e += BT) r.eC[e] = c.eC[e];
        __syncthreads();
    }
}

// State at the start of every chunk: S_{n+1} = Diag(eC) S_n + Kh^T (Ut - W S_n), per 64 value columns.
__global__ __launch_bounds__(BT) void bwd_states_kernel(KdaBwdArgs a) {
    __shared__ float tA[16][65], tB[16][65];
    const int DK = a.dk, DV = a.dv, nvs = DV / VS;
    const int bh = blockIdx.x / nvs, j0 = (blockIdx.x % nvs) * VS;
    float *S = a.scratch + (size_t)blockIdx.x * a.scratch_floats;   // [DK][VS]
    float *U = S + (size_t)DK * VS;                                  // [BC][VS]
    for (int e = threadIdx.x; e < DK * VS; e += BT) {
        const int i = e / VS, j = e % VS;
        S[e] = a.s0 ? a.s0[((size_t)bh * DK + i) * DV + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int n = 0; n < a.n_chunks; ++n) {
        float *Sn = a.states + ((size_t)bh * a.n_chunks + n) * DK * DV;
        for (int e = threadIdx.x; e < DK * VS; e += BT) Sn[(size_t)(e / VS) * DV + j0 + e % VS] = S[e];
        const Rec r = rec_at(a, bh, n);
        for (int e = threadIdx.x; e < BC * VS; e += BT) U[e] = r.Ut[(size_t)(e / VS) * DV + j0 + e % VS];
        __syncthreads();
        gemm<false, false>(U, VS, r.W, DK, S, VS, BC, VS, DK, -1.f, true, kNoMask, tA, tB);   // U = Ut - W S
        for (int e = threadIdx.x; e < DK * VS; e += BT) S[e] *= r.eC[e / VS];
        __syncthreads();
        gemm<true, false>(S, VS, r.Kh, DK, U, VS, DK, VS, BC, 1.f, true, kNoMask, tA, tB);    // S += Kh^T U
    }
    if (a.sT)
        for (int e = threadIdx.x; e < DK * VS; e += BT) a.sT[((size_t)bh * DK + e / VS) * DV + j0 + e % VS] = S[e];
}

// Reverse pass: dS' of every chunk (the gradient of the state after it) and dS0.
template <typename T>
__global__ __launch_bounds__(BT) void bwd_reverse_kernel(KdaBwdArgs a) {
    __shared__ float tA[16][65], tB[16][65];
    const int DK = a.dk, DV = a.dv, H = a.H, nvs = DV / VS;
    const int bh = blockIdx.x / nvs, j0 = (blockIdx.x % nvs) * VS, b = bh / H, h = bh % H;
    float *dS = a.scratch + (size_t)blockIdx.x * a.scratch_floats;   // [DK][VS]
    float *dSn = dS + (size_t)DK * VS;                               // [DK][VS]
    float *dU = dSn + (size_t)DK * VS;                               // [BC][VS]
    float *dO = dU + (size_t)BC * VS;                                // [BC][VS]
    const T *go = static_cast<const T *>(a.dO);
    for (int e = threadIdx.x; e < DK * VS; e += BT) {
        const int i = e / VS, j = e % VS;
        dS[e] = a.dsT ? a.dsT[((size_t)bh * DK + i) * DV + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int n = a.n_chunks - 1; n >= 0; --n) {
        float *dSp = a.dstates + ((size_t)bh * a.n_chunks + n) * DK * DV;
        for (int e = threadIdx.x; e < DK * VS; e += BT) dSp[(size_t)(e / VS) * DV + j0 + e % VS] = dS[e];
        const int t0 = n * BC, nr = min(BC, a.T - t0);
        for (int e = threadIdx.x; e < BC * VS; e += BT) {
            const int r = e / VS, j = e % VS;
            dO[e] = r < nr ? ld(go + (((size_t)b * a.T + t0 + r) * H + h) * DV + j0 + j) : 0.f;
        }
        __syncthreads();
        const Rec r = rec_at(a, bh, n);
        gemm<true, false>(dU, VS, r.Bq, BC, dO, VS, BC, VS, BC, 1.f, false, kNoMask, tA, tB);   // Bq^T dO
        gemm<false, false>(dU, VS, r.Kh, DK, dS, VS, BC, VS, DK, 1.f, true, kNoMask, tA, tB);   // + Kh dS'
        for (int e = threadIdx.x; e < DK * VS; e += BT) dSn[e] = r.eC[e / VS] * dS[e];
        __syncthreads();
        gemm<true, false>(dSn, VS, r.Qt, DK, dO, VS, DK, VS, BC, 1.f, true, kNoMask, tA, tB);   // + Qt^T dO
        gemm<true, false>(dSn, VS, r.W, DK, dU, VS, DK, VS, BC, -1.f, true, kNoMask, tA, tB);   // - W^T dU
        float *t = dS;
        dS = dSn;
        dSn = t;
    }
    if (a.ds0)
        for (int e = threadIdx.x; e < DK * VS; e += BT) a.ds0[((size_t)bh * DK + e / VS) * DV + j0 + e % VS] = dS[e];
}

// Gradients of one chunk's tokens.
template <typename T>
__global__ __launch_bounds__(BT) void bwd_intra_kernel(KdaBwdArgs a) {
    __shared__ float tA[16][65], tB[16][65];
    const int DK = a.dk, DV = a.dv, H = a.H, tid = threadIdx.x;
    float *s;
    const ChunkMats c = carve(a.scratch + (size_t)blockIdx.x * a.scratch_floats, DK, DV, &s);
    const size_t mk = (size_t)BC * DK, mv = (size_t)BC * DV, mc = (size_t)BC * BC;
    float *U = s; s += mv;
    float *dO = s; s += mv;
    float *dU = s; s += mv;
    float *dBq = s; s += mc;
    float *dQt = s; s += mk;
    float *dKh = s; s += mk;
    float *dW = s; s += mk;
    float *dTm = s; s += mc;
    float *P = s; s += mc;     // Tm^T dTm
    float *dM = s; s += mc;
    float *dX = s; s += mv;
    float *dY = s; s += mk;
    float *dKt = s; s += mk;
    float *dKd = s; s += mk;
    float *dG = s; s += mk;
    T *gq = static_cast<T *>(a.dq), *gk = static_cast<T *>(a.dk_out), *gv = static_cast<T *>(a.dv_out);
    T *ga = static_cast<T *>(a.dalpha), *gb = static_cast<T *>(a.dbeta);
    const T *go = static_cast<const T *>(a.dO), *al = static_cast<const T *>(a.alpha);
    const int items = a.B * H * a.n_chunks;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int bh = it / a.n_chunks, n = it % a.n_chunks, b = bh / H, h = bh % H;
        const int t0 = n * BC, nr = min(BC, a.T - t0);
        auto tok = [&](int r) { return ((size_t)b * a.T + t0 + r) * H + h; };
        chunk_forward<T>(a, c, bh, n, tA, tB);
        const float *Sn = a.states + ((size_t)bh * a.n_chunks + n) * DK * DV;
        const float *dSp = a.dstates + ((size_t)bh * a.n_chunks + n) * DK * DV;
        for (int e = tid; e < BC * DV; e += BT) {
            const int r = e / DV;
            U[e] = c.Ut[e];
            dO[e] = r < nr ? ld(go + tok(r) * DV + e % DV) : 0.f;
        }
        __syncthreads();
        gemm<false, false>(U, DV, c.W, DK, Sn, DV, BC, DV, DK, -1.f, true, kNoMask, tA, tB);        // U = Ut - W S
        gemm<true, false>(dU, DV, c.Bq, BC, dO, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);       // dU = Bq^T dO
        gemm<false, false>(dU, DV, c.Kh, DK, dSp, DV, BC, DV, DK, 1.f, true, kNoMask, tA, tB);      //    + Kh dS'
        gemm<false, true>(dBq, BC, dO, DV, U, DV, BC, BC, DV, 1.f, false, kLower, tA, tB);          // dBq
        gemm<false, true>(dQt, DK, dO, DV, Sn, DV, BC, DK, DV, 1.f, false, kNoMask, tA, tB);        // dQt = dO S^T
        gemm<false, false>(dQt, DK, dBq, BC, c.Kd, DK, BC, DK, BC, 1.f, true, kNoMask, tA, tB);     //     + dBq Kd
        gemm<false, true>(dKh, DK, U, DV, dSp, DV, BC, DK, DV, 1.f, false, kNoMask, tA, tB);        // dKh = U dS'^T
        gemm<false, true>(dW, DK, dU, DV, Sn, DV, BC, DK, DV, -1.f, false, kNoMask, tA, tB);        // dW = -dU S^T
        gemm<false, true>(dTm, BC, dU, DV, c.X, DV, BC, BC, DV, 1.f, false, kNoMask, tA, tB);       // dTm = dU X^T
        gemm<false, true>(dTm, BC, dW, DK, c.Y, DK, BC, BC, DK, 1.f, true, kNoMask, tA, tB);        //     + dW Y^T
        gemm<true, false>(P, BC, c.Tm, BC, dTm, BC, BC, BC, BC, 1.f, false, kNoMask, tA, tB);       // Tm^T dTm
        gemm<false, true>(dM, BC, P, BC, c.Tm, BC, BC, BC, BC, -1.f, false, kNoMask, tA, tB);       // dM
        gemm<true, false>(dX, DV, c.Tm, BC, dU, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);       // dX = Tm^T dU
        gemm<true, false>(dY, DK, c.Tm, BC, dW, DK, BC, DK, BC, 1.f, false, kNoMask, tA, tB);       // dY = Tm^T dW
        // dA = strict_lower(Diag(beta) dM), kept in dM's strict lower part (P reused for it)
        for (int e = tid; e < BC * BC; e += BT) {
            const int r = e / BC, s2 = e % BC;
            P[e] = s2 < r ? c.beta[r] * dM[e] : 0.f;
        }
        for (int e = tid; e < BC * DK; e += BT) dKt[e] = c.beta[e / DK] * dY[e];
        __syncthreads();
        gemm<false, false>(dKt, DK, P, BC, c.Kd, DK, BC, DK, BC, 1.f, true, kNoMask, tA, tB);       // + dA Kd
        gemm<true, false>(dKd, DK, P, BC, c.Kt, DK, BC, DK, BC, 1.f, false, kNoMask, tA, tB);       // dA^T Kt
        gemm<true, false>(dKd, DK, dBq, BC, c.Qt, DK, BC, DK, BC, 1.f, true, kNoMask, tA, tB);      // + dBq^T Qt
        // per-token outputs
        if (tid < BC && tid < nr) {
            const int r = tid;
            float db = 0.f;
            for (int s2 = 0; s2 < r; ++s2) db += dM[r * BC + s2] * c.A[r * BC + s2];
            for (int j = 0; j < DV; ++j) db += dX[r * DV + j] * c.V[r * DV + j];
            for (int ch = 0; ch < DK; ++ch) db += dY[r * DK + ch] * c.Kt[r * DK + ch];
            st(gb + tok(r), db);
        }
        for (int e = tid; e < BC * DV; e += BT) {
            const int r = e / DV;
            if (r < nr) st(gv + tok(r) * DV + e % DV, c.beta[r] * dX[e]);
        }
        for (int e = tid; e < BC * DK; e += BT) {
            const int r = e / DK, ch = e % DK;
            const float g = c.G[e], gc = logf(c.eC[ch]), gm = expf(g);
            if (r < nr) {
                st(gq + tok(r) * DK + ch, gm * dQt[e]);
                st(gk + tok(r) * DK + ch, gm * dKt[e] + dKd[e] / gm + expf(gc - g) * dKh[e]);
            }
            dG[e] = dQt[e] * c.Qt[e] + dKt[e] * c.Kt[e] - dKd[e] * c.Kd[e] - dKh[e] * c.Kh[e];
        }
        __syncthreads();
        // the last row's extra terms, then the reverse cumulative sum down the rows
        for (int ch = tid; ch < DK; ch += BT) {
            float extra = 0.f, sds = 0.f;
            for (int r = 0; r < BC; ++r) extra += dKh[r * DK + ch] * c.Kh[r * DK + ch];
            for (int j = 0; j < DV; ++j) sds += dSp[(size_t)ch * DV + j] * Sn[(size_t)ch * DV + j];
            // the chunk's last row is its last valid token: rows past the end contribute nothing
            const int last = nr - 1;
            dG[last * DK + ch] += extra + c.eC[ch] * sds;
            float run = 0.f;
            for (int r = last; r >= 0; --r) {
                run += dG[r * DK + ch];
                st(ga + tok(r) * DK + ch, run / ld(al + tok(r) * DK + ch));
            }
        }
        __syncthreads();
    }
}

}  // namespace

size_t kda_bwd_scratch_floats(int dk, int dv) {
    const size_t mk = (size_t)BC * dk, mv = (size_t)BC * dv, mc = (size_t)BC * BC;
    // ChunkMats + the intra kernel's temporaries (the largest user)
    const size_t chunk = 9 * mk + 4 * mv + 3 * mc + BC + dk;
    const size_t intra = 3 * mv + 4 * mc + 6 * mk + mv + mk;
    return chunk + intra + 64;
}

size_t kda_bwd_rec_floats(int dk, int dv) { return 3 * (size_t)BC * dk + (size_t)BC * dv + (size_t)BC * BC + dk; }

hipError_t launch_kda_backward(KdaBwdArgs a, bool bf16, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    const int items = a.B * a.H * a.n_chunks;
    const int g = items < kBwdBlocks ? items : kBwdBlocks;
    const int ordered = a.B * a.H * (a.dv / VS);
    if (bf16) {
        hipLaunchKernelGGL(bwd_prep_kernel<bf16_t>, dim3(g), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_states_kernel, dim3(ordered), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_reverse_kernel<bf16_t>, dim3(ordered), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_intra_kernel<bf16_t>, dim3(g), dim3(BT), 0, stream, a);
    } else {
        hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(g), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_states_kernel, dim3(ordered), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_reverse_kernel<float>, dim3(ordered), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_intra_kernel<float>, dim3(g), dim3(BT), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kdaconv
