// Backward pass of the KDA scan (gradients of q, k, v, alpha, beta and the
// initial state, given those of o and the final state), chunk by chunk.
//
// Per chunk of C = 64 rows r (G_r = sum_{u<=r} log2 alpha_u per key channel,
// gam = 2^G, gC = G of the last row, e(r, s) = 2^(G_r - G_s) <= 1 for s <= r), the
// forward is regrouped as
//   Kt = gam K, Qt = gam Q, Kh = 2^(gC - G) K,
//   A[r][s] = sum_c K[r][c] K[s][c] e(r, s, c) (s < r), Bq[r][s] = sum_c Q[r][c] K[s][c] e(r, s, c) (s <= r),
//   Tm = (I + Diag(beta) A)^-1, X = Diag(beta) V, Y = Diag(beta) Kt, W = Tm Y, Ut = Tm X
//   (formed as (Tm Diag(beta)) Kt and (Tm Diag(beta)) V),
//   U = Ut - W S, O = Qt S + Bq U, S' = Diag(2^gC) S + Kh^T U
// and its adjoint, for dO and dS' (the gradient of the state after the chunk), is
//   dU = Bq^T dO + Kh dS',  dS = Qt^T dO + Diag(2^gC) dS' - W^T dU,
//   dBq = lower(dO U^T), dQt = dO S^T, dKh = U dS'^T, dW = -dU S^T,
//   dTm = dU X^T + dW Y^T, dM = -Tm^T dTm Tm^T, dA = strict_lower(Diag(beta) dM),
//   dX = Tm^T dU, dY = Tm^T dW, dbeta = rowsum(dM A) + rowsum(dX V) + rowsum(dY Kt), dV = Diag(beta) dX,
//   dQ  = gam dQt + R(dBq, K),                       R(P, Y)[r] = sum_{s<=r} P[r][s] Y[s] e(r, s)
//   dKx = gam Diag(beta) dY + R(dA, K),  dKy = C(dA, K) + C(dBq, Q),  C(P, X)[s] = sum_{r>=s} P[r][s] X[r] e(r, s)
//   dKh' = 2^(gC - G) dKh,  dK = dKx + dKy + dKh',
//   dG = Q dQ + K (dKx - dKy - dKh')  (+ on the last row: colsum(dKh Kh) + 2^gC rowsum(dS' S)),
//   dlog alpha = reverse cumulative sum of dG over the chunk (natural-log units), dalpha = dlog alpha / alpha.
// (dQ, dKx, dKy and dKh' are the gradients reaching q and k through Qt, Kt, the
// column side of A and Bq, and Kh; G enters each of them through its decay.)
// The decayed products A, Bq, R and C split e(r, s) at a row between r and s
// (tri_form2, tri_rows2, tri_cols2 below), so no factor exceeds the inverse of an
// 8-token decay: the range is the forward's.
//
// Three launches, all fp32 inside:
//   1. bwd_prep:    per (batch, head, chunk), in parallel: Qt, Kh, A, Bq, Tm, W, Ut, exp(gC).
//   2. bwd_ordered: two independent passes side by side, per (batch, head, 16 value
//                   columns): in chunk order the state at the start of every chunk,
//                   and in reverse chunk order dS' of every chunk and the gradient of
//                   the initial state.
//   3. bwd_intra:   per (batch, head, chunk), in parallel: the gradients of the
//                   chunk's tokens.
// The dense products run through one LDS-tiled fp32 routine (64 x 64 output
// tiles on the fp32 matrix cores; two-output forms for pairs that share an
// operand), and products that share operands are formed in one pass
// (tri_form2, tri_rows2, tri_cols2, gemm2_nt, gemm2_nn); all arithmetic is fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace kdaconv {
namespace {

constexpr int BC = kChunk;      // rows per chunk
constexpr int BT = 256;         // threads per workgroup

// ---- small dense helpers (all threads of the workgroup take part) ------------

enum Mask { kNoMask = 0, kLower = 1, kStrictLower = 2 };

// C[m][n] = scale * sum_k op(A)[m][k] op(B)[k][n]  (+ C when acc), for m < M, n < N;
// op(A)[m][k] = TA ? A[k*lda + m] : A[m*lda + k]; op(B)[k][n] = TB ? B[n*ldb + k] : B[k*ldb + n].
// M, N multiples of 64, K a multiple of 32 and at most 128, leading dimensions multiples
// of 4 and 16-byte aligned operands.  Per 64 x 64 output tile, K is walked in steps of
// kKc rows: the panels of step j+1 (float4 loads into registers, two pieces per thread
// and operand) are in flight while step j is computed from LDS, and the steps alternate
// between two LDS buffers (tA[k][m], tB[k][n]), so one barrier per step suffices.  The
// products run on the fp32 matrix cores.  The mask zeroes the result above the diagonal (kLower) or
// on and above it (kStrictLower).  Ends with a barrier.
constexpr int kPanel = 128;   // rows of the LDS panel area (two buffers of kKc rows in use)
constexpr int kPs = 68;       // panel row stride (64 + 4)
constexpr int kKc = 32;       // K rows per pipelined step
static_assert(kKc * 64 == 8 * BT, "two float4 pieces per thread and operand per step");

__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// This thread's pieces e = tid, tid + BT of the kKc x 64 panels of op(A) (columns m0..) and
// op(B) (columns n0..) at K rows k0..
template <bool TA, bool TB>
__device__ __forceinline__ void panel_fetch(const float *A, int lda, const float *B, int ldb, int m0, int n0, int k0,
                                            float4 (&va)[2], float4 (&vb)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = threadIdx.x + BT * i;
        va[i] = TA ? ld4f(A + (size_t)(k0 + e / 16) * lda + m0 + 4 * (e % 16))
                   : ld4f(A + (size_t)(m0 + e / 8) * lda + k0 + 4 * (e % 8));
        vb[i] = TB ? ld4f(B + (size_t)(n0 + e / 8) * ldb + k0 + 4 * (e % 8))
                   : ld4f(B + (size_t)(k0 + e / 16) * ldb + n0 + 4 * (e % 16));
    }
}
template <bool TA, bool TB>
__device__ __forceinline__ void panel_store(float (*pa)[kPs], float (*pb)[kPs], const float4 (&va)[2],
                                            const float4 (&vb)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = threadIdx.x + BT * i;
        if (TA) {
            *reinterpret_cast<float4 *>(&pa[e / 16][4 * (e % 16)]) = va[i];
        } else {
            const int mm = e / 8, q = e % 8;
            pa[4 * q][mm] = va[i].x;
            pa[4 * q + 1][mm] = va[i].y;
            pa[4 * q + 2][mm] = va[i].z;
            pa[4 * q + 3][mm] = va[i].w;
        }
        if (TB) {
            const int nn = e / 8, q = e % 8;
            pb[4 * q][nn] = vb[i].x;
            pb[4 * q + 1][nn] = vb[i].y;
            pb[4 * q + 2][nn] = vb[i].z;
            pb[4 * q + 3][nn] = vb[i].w;
        } else {
            *reinterpret_cast<float4 *>(&pb[e / 16][4 * (e % 16)]) = vb[i];
        }
    }
}

template <bool TA, bool TB>
__device__ __noinline__ void gemm(float *C, int ldc, const float *A, int lda, const float *B, int ldb, int M, int N, int K,
                     float scale, bool acc, Mask mask, float (*tA)[kPs], float (*tB)[kPs]) {
    // wave w forms the 32 x 32 quarter (rows 32 (w / 2) .., columns 32 (w % 2) ..) of each
    // tile as 2 x 2 blocks of 16 x 16 on the fp32 matrix cores: per 4-deep k step, lane l
    // supplies A[l%16][k + l/16] and B[k + l/16][l%16] of each block and holds rows
    // 4 (l/16) + i, column l%16 of each result
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const int wm = 32 * (wave / 2), wn = 32 * (wave % 2);
    const int nk = K / kKc;
    for (int m0 = 0; m0 < M; m0 += 64)
        for (int n0 = 0; n0 < N; n0 += 64) {
            float4 va[2], vb[2];
            panel_fetch<TA, TB>(A, lda, B, ldb, m0, n0, 0, va, vb);
            f32x4_t c[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
            for (int kc = 0; kc < nk; ++kc) {
                float(*pa)[kPs] = tA + (kc & 1) * kKc;
                float(*pb)[kPs] = tB + (kc & 1) * kKc;
                panel_store<TA, TB>(pa, pb, va, vb);
                __syncthreads();
                // the next step's panels (the last step fetches its own again: no branch, so
                // the loads need not complete before the products below)
                panel_fetch<TA, TB>(A, lda, B, ldb, m0, n0, min(kc + 1, nk - 1) * kKc, va, vb);
#pragma unroll
                for (int k = 0; k < kKc; k += 4) {
                    const float a0 = pa[k + g][wm + l16], a1 = pa[k + g][wm + 16 + l16];
                    const float b0 = pb[k + g][wn + l16], b1 = pb[k + g][wn + 16 + l16];
                    c[0][0] = mma4(a0, b0, c[0][0]);
                    c[0][1] = mma4(a0, b1, c[0][1]);
                    c[1][0] = mma4(a1, b0, c[1][0]);
                    c[1][1] = mma4(a1, b1, c[1][1]);
                }
            }
#pragma unroll
            for (int bm = 0; bm < 2; ++bm)
#pragma unroll
                for (int bn = 0; bn < 2; ++bn)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = m0 + wm + 16 * bm + 4 * g + i, n = n0 + wn + 16 * bn + l16;
                        float x = scale * c[bm][bn][i];
                        if ((mask == kLower && n > m) || (mask == kStrictLower && n >= m)) x = 0.f;
                        float *p = C + (size_t)m * ldc + n;
                        *p = acc ? *p + x : x;
                    }
            __syncthreads();
        }
}

// C1 = s1 A1 B^T and C2 = s2 A2 B^T (A1, A2 row-major M x K, B row-major N x K, as gemm's
// TA = false, TB = true): two products that share B^T, so each step stages B's panel once for
// both.  The second A's panels use the other half of the A panel area (rows 2 kKc ..).
__device__ __noinline__ void gemm2_nt(float *C1, float s1, const float *A1, float *C2, float s2, const float *A2,
                                      int lda, const float *B, int ldb, int ldc, int M, int N, int K,
                                      float (*tA)[kPs], float (*tB)[kPs]) {
    static_assert(4 * kKc <= kPanel, "two double-buffered A panels fit the panel area");
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const int wm = 32 * (wave / 2), wn = 32 * (wave % 2);
    const int nk = K / kKc;
    // this thread's pieces of the second A's kKc x 64 panel (as panel_fetch / panel_store
    // do for A with TA = false)
    auto fetch2 = [&](int m0, int k0, float4 (&v)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = threadIdx.x + BT * i;
            v[i] = ld4f(A2 + (size_t)(m0 + e / 8) * lda + k0 + 4 * (e % 8));
        }
    };
    auto store2 = [&](float (*pa)[kPs], const float4 (&v)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = threadIdx.x + BT * i, mm = e / 8, q = e % 8;
            pa[4 * q][mm] = v[i].x;
            pa[4 * q + 1][mm] = v[i].y;
            pa[4 * q + 2][mm] = v[i].z;
            pa[4 * q + 3][mm] = v[i].w;
        }
    };
    for (int m0 = 0; m0 < M; m0 += 64)
        for (int n0 = 0; n0 < N; n0 += 64) {
            float4 va[2], vb[2], va2[2];
            panel_fetch<false, true>(A1, lda, B, ldb, m0, n0, 0, va, vb);
            fetch2(m0, 0, va2);
            f32x4_t c1[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
            f32x4_t c2[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
            for (int kc = 0; kc < nk; ++kc) {
                float(*pa)[kPs] = tA + (kc & 1) * kKc;
                float(*pa2)[kPs] = tA + 2 * kKc + (kc & 1) * kKc;
                float(*pb)[kPs] = tB + (kc & 1) * kKc;
                panel_store<false, true>(pa, pb, va, vb);
                store2(pa2, va2);
                __syncthreads();
                // the next step's panels (the last step fetches its own again: no branch)
                const int k1 = min(kc + 1, nk - 1) * kKc;
                panel_fetch<false, true>(A1, lda, B, ldb, m0, n0, k1, va, vb);
                fetch2(m0, k1, va2);
#pragma unroll 4
                for (int k = 0; k < kKc; k += 4) {
                    const float b0 = pb[k + g][wn + l16], b1 = pb[k + g][wn + 16 + l16];
                    const float a0 = pa[k + g][wm + l16], a1 = pa[k + g][wm + 16 + l16];
                    const float d0 = pa2[k + g][wm + l16], d1 = pa2[k + g][wm + 16 + l16];
                    c1[0][0] = mma4(a0, b0, c1[0][0]);
                    c1[0][1] = mma4(a0, b1, c1[0][1]);
                    c1[1][0] = mma4(a1, b0, c1[1][0]);
                    c1[1][1] = mma4(a1, b1, c1[1][1]);
                    c2[0][0] = mma4(d0, b0, c2[0][0]);
                    c2[0][1] = mma4(d0, b1, c2[0][1]);
                    c2[1][0] = mma4(d1, b0, c2[1][0]);
                    c2[1][1] = mma4(d1, b1, c2[1][1]);
                }
            }
#pragma unroll
            for (int bm = 0; bm < 2; ++bm)
#pragma unroll
                for (int bn = 0; bn < 2; ++bn)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const size_t o = (size_t)(m0 + wm + 16 * bm + 4 * g + i) * ldc + n0 + wn + 16 * bn + l16;
                        C1[o] = s1 * c1[bm][bn][i];
                        C2[o] = s2 * c2[bm][bn][i];
                    }
            __syncthreads();
        }
}

// C1 = A B1 and C2 = A B2 (A row-major M x K, B1, B2 row-major K x N, as gemm's TA = false,
// TB = false; both C with leading dimension ldc): two products that share A, so each step
// stages A's panel once for both.  The second B's panels use the other half of the B panel
// area (rows 2 kKc ..).
__device__ __noinline__ void gemm2_nn(float *C1, float *C2, int ldc, const float *A, int lda, const float *B1,
                                      const float *B2, int ldb, int M, int N, int K, float (*tA)[kPs],
                                      float (*tB)[kPs]) {
    static_assert(4 * kKc <= kPanel, "two double-buffered B panels fit the panel area");
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const int wm = 32 * (wave / 2), wn = 32 * (wave % 2);
    const int nk = K / kKc;
    // this thread's pieces of the second B's kKc x 64 panel (as panel_fetch / panel_store
    // do for B with TB = false)
    auto fetch2 = [&](int n0, int k0, float4 (&v)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = threadIdx.x + BT * i;
            v[i] = ld4f(B2 + (size_t)(k0 + e / 16) * ldb + n0 + 4 * (e % 16));
        }
    };
    auto store2 = [&](float (*pb)[kPs], const float4 (&v)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = threadIdx.x + BT * i;
            *reinterpret_cast<float4 *>(&pb[e / 16][4 * (e % 16)]) = v[i];
        }
    };
    for (int m0 = 0; m0 < M; m0 += 64)
        for (int n0 = 0; n0 < N; n0 += 64) {
            float4 va[2], vb[2], vb2[2];
            panel_fetch<false, false>(A, lda, B1, ldb, m0, n0, 0, va, vb);
            fetch2(n0, 0, vb2);
            f32x4_t c1[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
            f32x4_t c2[2][2] = {{zero4(), zero4()}, {zero4(), zero4()}};
            for (int kc = 0; kc < nk; ++kc) {
                float(*pa)[kPs] = tA + (kc & 1) * kKc;
                float(*pb)[kPs] = tB + (kc & 1) * kKc;
                float(*pb2)[kPs] = tB + 2 * kKc + (kc & 1) * kKc;
                panel_store<false, false>(pa, pb, va, vb);
                store2(pb2, vb2);
                __syncthreads();
                // the next step's panels (the last step fetches its own again: no branch)
                const int k1 = min(kc + 1, nk - 1) * kKc;
                panel_fetch<false, false>(A, lda, B1, ldb, m0, n0, k1, va, vb);
                fetch2(n0, k1, vb2);
#pragma unroll 2
                for (int k = 0; k < kKc; k += 4) {
                    const float a0 = pa[k + g][wm + l16], a1 = pa[k + g][wm + 16 + l16];
                    const float b0 = pb[k + g][wn + l16], b1 = pb[k + g][wn + 16 + l16];
                    const float d0 = pb2[k + g][wn + l16], d1 = pb2[k + g][wn + 16 + l16];
                    c1[0][0] = mma4(a0, b0, c1[0][0]);
                    c1[0][1] = mma4(a0, b1, c1[0][1]);
                    c1[1][0] = mma4(a1, b0, c1[1][0]);
                    c1[1][1] = mma4(a1, b1, c1[1][1]);
                    c2[0][0] = mma4(a0, d0, c2[0][0]);
                    c2[0][1] = mma4(a0, d1, c2[0][1]);
                    c2[1][0] = mma4(a1, d0, c2[1][0]);
                    c2[1][1] = mma4(a1, d1, c2[1][1]);
                }
            }
#pragma unroll
            for (int bm = 0; bm < 2; ++bm)
#pragma unroll
                for (int bn = 0; bn < 2; ++bn)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const size_t o = (size_t)(m0 + wm + 16 * bm + 4 * g + i) * ldc + n0 + wn + 16 * bn + l16;
                        C1[o] = c1[bm][bn][i];
                        C2[o] = c2[bm][bn][i];
                    }
            __syncthreads();
        }
}

// ---- decayed triangular products ---------------------------------------------------
//
// Row r of a chunk sees an earlier row s <= r of channel c through the decay
// e(r, s, c) = 2^(G[r][c] - G[s][c]) <= 1.  Formed as 2^G times 2^-G over the whole chunk,
// the second factor leaves the fp32 range once a chunk decays by more than 2^-126.  Here
// the factor is split at a reference row between r and s, with the rows in 16-row blocks:
//   * r in block i, s in an earlier block j: the last row of block i - 1 (tri_form2,
//     tri_rows2) or of block j (tri_cols2) lies between them, so both halves are decays;
//   * r and s in one block: its row 7, so each half is at most the inverse of an
//     8-token decay (the forward chunk transform's bound).
// X, Y, G, Z are fp32 row-major [BC][DK] and P, C [BC][BC], in global memory (the
// workgroup's scratch or the chunk's record); DK is 64 or 128.  The products run on
// v_mfma_f32_16x16x4_f32: per step lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// the result leaves rows 4 (l/16) + i, column l%16 in lane l; the step's contraction
// index l/16 stands for index 4 (l/16) + v of a 16-wide block, v the step, so each lane
// reads 4 consecutive elements.  Every thread of the workgroup calls these; each ends
// with a barrier.

// 2^x on the hardware exponential (about 1 ulp; results below 2^-126, negligible
// beside the terms they join, come out as zero).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// A matrix of the decayed products (global memory) read and written through a buffer
// resource: its base in scalar registers (every lane passes the same pointer), the lane's
// part of an address in one vector register and the constant part (a row offset known at
// compile time) as an immediate or scalar offset, so the many loads of a product need
// no 64-bit address each.  Offsets are in elements.
struct GMat {
    __amdgpu_buffer_rsrc_t rs;
    __device__ __forceinline__ GMat(const float *p, int n) {
        // readfirstlane returns a signed int: widen each half through uint32_t, or a low
        // word with bit 31 set would sign-extend over the high word
        const uint64_t a = reinterpret_cast<uint64_t>(p);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
        const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
        rs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), 0, 4 * n, kBufWord3);
    }
    __device__ __forceinline__ float at(int lane_off, int off) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane_off, 4 * off, 0));
    }
    __device__ __forceinline__ float4 at4(int lane_off, int off) const {
        return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * lane_off, 4 * off, 0));
    }
    __device__ __forceinline__ void put(float x, int lane_off, int off) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, 4 * lane_off, 4 * off, 0);
    }
};

// The 16 block pairs (i, j) of a 64 x 64 result: the 10 on and below the diagonal first,
// row by row, then the 6 above it (zero), so that the four waves share the work evenly.
__device__ __forceinline__ void block_pair(int p, int &i, int &j) {
    if (p < 10) {
        i = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
        j = p - i * (i + 1) / 2;
    } else {
        const int q = p - 10;
        i = q < 3 ? 0 : q < 5 ? 1 : 2;
        j = i + 1 + q - (i == 0 ? 0 : i == 1 ? 3 : 5);
    }
}

// A[r][s] = sum_c K[r][c] K[s][c] e(r, s, c) for s < r and Bq[r][s] = sum_c Q[r][c] K[s][c]
// e(r, s, c) for s <= r, 0 above: one pass, since both read the same rows of K (as the
// right factor) and of G, so the decayed right factor and the left decay are formed once.
// Every load of a block pair is issued before its products.
template <int DK>
__device__ __noinline__ void tri_form2_k(float *Ac, float *Bc, const float *K, const float *Q, const float *G) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const GMat Am(Ac, BC * BC), Bm(Bc, BC * BC), Km(K, BC * DK), Qm(Q, BC * DK), Gm(G, BC * DK);
    constexpr int NU = DK / 16;
    for (int p = wave; p < 16; p += BT / 64) {
        int i, j;
        block_pair(p, i, j);
        f32x4_t acc = zero4(), bcc = zero4();
        if (j <= i) {
            const int ref = j < i ? 16 * i - 1 : 16 * i + 7;
            const int xo = (16 * i + l16) * DK + 4 * g, yo = (16 * j + l16) * DK + 4 * g, ro = ref * DK + 4 * g;
            float4 kx[NU], qx[NU], xg[NU], yv[NU], yg[NU], rg[NU];
#pragma unroll
            for (int t = 0; t < NU; ++t) {
                kx[t] = Km.at4(xo, 16 * t);
                qx[t] = Qm.at4(xo, 16 * t);
                xg[t] = Gm.at4(xo, 16 * t);
                yv[t] = Km.at4(yo, 16 * t);
                yg[t] = Gm.at4(yo, 16 * t);
                rg[t] = Gm.at4(ro, 16 * t);
            }
#pragma unroll
            for (int t = 0; t < NU; ++t) {
                const float ex[4] = {ex2(xg[t].x - rg[t].x), ex2(xg[t].y - rg[t].y), ex2(xg[t].z - rg[t].z),
                                     ex2(xg[t].w - rg[t].w)};
                const float y[4] = {yv[t].x * ex2(rg[t].x - yg[t].x), yv[t].y * ex2(rg[t].y - yg[t].y),
                                    yv[t].z * ex2(rg[t].z - yg[t].z), yv[t].w * ex2(rg[t].w - yg[t].w)};
                const float kk[4] = {kx[t].x, kx[t].y, kx[t].z, kx[t].w};
                const float qq[4] = {qx[t].x, qx[t].y, qx[t].z, qx[t].w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc = mma4(kk[v] * ex[v], y[v], acc);
                    bcc = mma4(qq[v] * ex[v], y[v], bcc);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 16 * i + 4 * g + q, s2 = 16 * j + l16;
            // selects, not products: inside a diagonal block the terms above the
            // diagonal may overflow
            Am.put(s2 >= r ? 0.f : acc[q], r * BC + s2, 0);
            Bm.put(s2 > r ? 0.f : bcc[q], r * BC + s2, 0);
        }
    }
    __syncthreads();
}

// Z1[r][c] = sum_{s <= r} P1[r][s] Y[s][c] e(r, s, c) and Z2 the same with P2 (P1, P2 zero
// above their diagonals): the two row-side products that share Y, so the decayed operand
// Y[s][c] e(ref, s, c) is formed once for both.  Per 16-column tile, a lane reads its 16 rows
// of Y and G once (rows 16 j + 4 (l/16) + v: the contraction rows of every block j and, the
// same rows, its outputs).
template <int DK>
__device__ __noinline__ void tri_rows2_k(float *Z1, const float *P1, float *Z2, const float *P2, const float *Y,
                                         const float *G) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const GMat Z1m(Z1, BC * DK), Z2m(Z2, BC * DK), P1m(P1, BC * BC), P2m(P2, BC * BC), Ym(Y, BC * DK),
        Gm(G, BC * DK);
#pragma unroll 1
    for (int n = wave; n < DK / 16; n += BT / 64) {
        const int c = 16 * n + l16, lo = 4 * g * DK + c;   // the lane's row 4 g, column c
        float yv[16], gv[16], gm[4], ge[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                yv[4 * j + v] = Ym.at(lo, (16 * j + v) * DK);
                gv[4 * j + v] = Gm.at(lo, (16 * j + v) * DK);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gm[i] = Gm.at(c, (16 * i + 7) * DK);
            ge[i] = i ? Gm.at(c, (16 * i - 1) * DK) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 p1[4], p2[4];
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                p1[j] = P1m.at4(l16 * BC + 4 * g, 16 * i * BC + 16 * j);
                p2[j] = P2m.at4(l16 * BC + 4 * g, 16 * i * BC + 16 * j);
            }
            f32x4_t off1 = zero4(), dia1 = zero4(), off2 = zero4(), dia2 = zero4();
#pragma unroll
            for (int j = 0; j <= i; ++j) {
                const float gref = j < i ? ge[i] : gm[i];
                float bv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) bv[v] = yv[4 * j + v] * ex2(gref - gv[4 * j + v]);
                f32x4_t &t1 = j < i ? off1 : dia1;
                f32x4_t &t2 = j < i ? off2 : dia2;
                t1 = mma4(p1[j].x, bv[0], t1);
                t1 = mma4(p1[j].y, bv[1], t1);
                t1 = mma4(p1[j].z, bv[2], t1);
                t1 = mma4(p1[j].w, bv[3], t1);
                t2 = mma4(p2[j].x, bv[0], t2);
                t2 = mma4(p2[j].y, bv[1], t2);
                t2 = mma4(p2[j].z, bv[2], t2);
                t2 = mma4(p2[j].w, bv[3], t2);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float gr = gv[4 * i + q], edia = ex2(gr - gm[i]), eoff = i ? ex2(gr - ge[i]) : 0.f;
                float z1 = edia * dia1[q], z2 = edia * dia2[q];
                if (i) {
                    z1 += eoff * off1[q];
                    z2 += eoff * off2[q];
                }
                const int ro = (16 * i + q) * DK;
                Z1m.put(z1, lo, ro);
                Z2m.put(z2, lo, ro);
            }
        }
    }
    __syncthreads();
}

// Z[s][c] = sum_{r >= s} (P1[r][s] X1[r][c] + P2[r][s] X2[r][c]) e(r, s, c) (P1, P2 zero above
// their diagonals): the two column-side products that accumulate into one output, so the
// decay factor e(r, ref, c) is formed once for both and Z is written once.  Per 16-column
// tile, the lane reads its 16 rows of X1, X2 and G once, and per output block column j its
// P1 and P2 entries of the block pairs (i >= j, j) just before their products.
// (inlined into its one caller: as a call it would need more scalar registers than a callee
// may use without saving the caller's)
template <int DK>
__device__ __forceinline__ void tri_cols2_k(float *Z, const float *P1, const float *X1, const float *P2, const float *X2,
                                         const float *G) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    const GMat Zm(Z, BC * DK), P1m(P1, BC * BC), P2m(P2, BC * BC), X1m(X1, BC * DK), X2m(X2, BC * DK),
        Gm(G, BC * DK);
#pragma unroll 1
    for (int n = wave; n < DK / 16; n += BT / 64) {
        const int c = 16 * n + l16, lo = 4 * g * DK + c;
        float x1[16], x2[16], gv[16], gm[4], ge[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                x1[4 * i + v] = X1m.at(lo, (16 * i + v) * DK);
                x2[4 * i + v] = X2m.at(lo, (16 * i + v) * DK);
                gv[4 * i + v] = Gm.at(lo, (16 * i + v) * DK);
            }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gm[j] = Gm.at(c, (16 * j + 7) * DK);
            ge[j] = Gm.at(c, (16 * j + 15) * DK);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float pa1[4][4], pa2[4][4];   // [i][v] = P[16 i + 4 g + v][16 j + l16], i >= j
#pragma unroll
            for (int i = j; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    pa1[i][v] = P1m.at(4 * g * BC + l16, (16 * i + v) * BC + 16 * j);
                    pa2[i][v] = P2m.at(4 * g * BC + l16, (16 * i + v) * BC + 16 * j);
                }
            f32x4_t off = zero4(), dia = zero4();
#pragma unroll
            for (int i = j; i < 4; ++i) {
                const float gref = i > j ? ge[j] : gm[j];
                f32x4_t &t = i > j ? off : dia;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float e = ex2(gv[4 * i + v] - gref);
                    t = mma4(pa1[i][v], x1[4 * i + v] * e, t);
                    t = mma4(pa2[i][v], x2[4 * i + v] * e, t);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float gs = gv[4 * j + q];
                float z = ex2(gm[j] - gs) * dia[q];
                if (j < 3) z += ex2(ge[j] - gs) * off[q];
                Zm.put(z, lo, (16 * j + q) * DK);
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void tri_form2(float *Ac, float *Bc, const float *K, const float *Q, const float *G, int DK) {
    if (DK == 128)
        tri_form2_k<128>(Ac, Bc, K, Q, G);
    else
        tri_form2_k<64>(Ac, Bc, K, Q, G);
}
__device__ __forceinline__ void tri_rows2(float *Z1, const float *P1, float *Z2, const float *P2, const float *Y,
                                          const float *G, int DK) {
    if (DK == 128)
        tri_rows2_k<128>(Z1, P1, Z2, P2, Y, G);
    else
        tri_rows2_k<64>(Z1, P1, Z2, P2, Y, G);
}
__device__ __forceinline__ void tri_cols2(float *Z, const float *P1, const float *X1, const float *P2, const float *X2,
                                          const float *G, int DK) {
    if (DK == 128)
        tri_cols2_k<128>(Z, P1, X1, P2, X2, G);
    else
        tri_cols2_k<64>(Z, P1, X1, P2, X2, G);
}

__device__ __forceinline__ float ld(const float *p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t *p) { return (float)*p; }
__device__ __forceinline__ void st(float *p, float x) { *p = x; }
__device__ __forceinline__ void st(bf16_t *p, float x) { *p = (bf16_t)x; }

// Per-chunk matrices rebuilt from the inputs (fp32, row-major, in the
// workgroup's scratch): the chunk's rows past the stream's end are zero.
struct ChunkMats {
    float *Q, *K, *V, *G, *Kt, *Qt, *Kh, *A, *Bq, *Tm, *TmB, *W, *Ut;   // TmB = Tm Diag(beta)
    float *beta, *eC;   // [BC], [DK]
};

// 8 consecutive elements as fp32.
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16_t *p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}

// rows x cols (cols a multiple of 8) of token-major input src (row r at src + r * stride)
// into dst (fp32, row-major, ld = cols); rows >= nr are zero.  Every thread issues the
// loads of 4 pieces of 8 elements before storing any of them.
template <typename T, typename D>
__device__ void stage_rows(D *dst, const T *src, size_t stride, int rows, int cols, int nr) {
    const int c8 = cols / 8, np = rows * c8;
    for (int p0 = 0; p0 < np; p0 += 4 * BT) {
        float x[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = min(p0 + (int)threadIdx.x + BT * i, np - 1), r = p / c8;
            ld8(src + (size_t)min(r, nr - 1) * stride + 8 * (p % c8), x[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = p0 + threadIdx.x + BT * i;
            if (p < np) {
                const int r = p / c8;
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[r * cols + 8 * (p % c8) + j] = r < nr ? x[i][j] : 0.f;
            }
        }
    }
}

// FULL: the whole transform.  Otherwise only what the gradient kernel needs beyond the
// chunk's record (Q, K, V, beta, G, Kt): Qt, Kh, A, Bq, Tm, W, Ut and 2^gC are already
// there (c points at them) from the records pass.  G is in log2 units.
template <typename T, bool FULL>
__device__ void chunk_forward(const KdaBwdArgs &a, const ChunkMats &c, int bh, int n, float (*tA)[kPs],
                              float (*tB)[kPs]) {
    const int DK = a.dk, DV = a.dv, H = a.H, tid = threadIdx.x;
    const int b = bh / H, h = bh % H, t0 = n * BC, nr = min(BC, a.T - t0);
    const size_t tok0 = ((size_t)b * a.T + t0) * H + h;   // token t0, head h
    const T *q = static_cast<const T *>(a.q), *k = static_cast<const T *>(a.k), *v = static_cast<const T *>(a.v);
    const T *al = static_cast<const T *>(a.alpha), *be = static_cast<const T *>(a.beta);
    float *lw = &tA[0][0];   // the panel area as scratch: 2 * kPanel * kPs floats (tB follows tA)
    stage_rows(c.V, v + tok0 * DV, (size_t)H * DV, BC, DV, nr);
    stage_rows(lw, al + tok0 * DK, (size_t)H * DK, BC, DK, nr);   // alpha (rows past the end: 0, unused)
    if (tid < BC) c.beta[tid] = tid < nr ? ld(be + tok0 + (size_t)tid * H) : 0.f;
    __syncthreads();
    // G: cumulative sum of log2 alpha down the rows (rows past the end add 0), in LDS
    for (int ch = tid; ch < DK; ch += BT) {
        float g = 0.f;
        for (int r = 0; r < BC; ++r) {
            if (r < nr) g += log2f(lw[r * DK + ch]);
            lw[r * DK + ch] = g;
        }
        if (FULL) c.eC[ch] = exp2f(g);
        lw[BC * DK + ch] = g;   // gC
    }
    __syncthreads();
    {
        float *__restrict__ Gg = c.G;
        float *__restrict__ Kt = c.Kt;
        float *__restrict__ Kr = c.K;
        float *__restrict__ Qr = c.Q;
        float *__restrict__ Qt = c.Qt;
        float *__restrict__ Kh = c.Kh;
        // q and k straight from the inputs (rows past the end read the first row, used as zeros)
        const T *__restrict__ kin = k + tok0 * DK;
        const T *__restrict__ qin = q + tok0 * DK;
        for (int e4 = tid; e4 < BC * DK / 4; e4 += BT) {
            const int e = 4 * e4, ch = e % DK, r = e / DK;
            const size_t src = (size_t)(r < nr ? r : 0) * H * DK + ch;
            float kv[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
            ld4(kin + src, kv);
            ld4(qin + src, qv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kv[i] = r < nr ? kv[i] : 0.f;
                qv[i] = r < nr ? qv[i] : 0.f;
            }
            float g4[4], kt[4], qt[4], kh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g = lw[e + i], gm = exp2f(g);
                g4[i] = g;
                kt[i] = gm * kv[i];
                qt[i] = gm * qv[i];
                kh[i] = exp2f(lw[BC * DK + ch + i] - g) * kv[i];
            }
            *reinterpret_cast<float4 *>(Gg + e) = make_float4(g4[0], g4[1], g4[2], g4[3]);
            *reinterpret_cast<float4 *>(Kt + e) = make_float4(kt[0], kt[1], kt[2], kt[3]);
            *reinterpret_cast<float4 *>(Kr + e) = make_float4(kv[0], kv[1], kv[2], kv[3]);
            *reinterpret_cast<float4 *>(Qr + e) = make_float4(qv[0], qv[1], qv[2], qv[3]);
            if (FULL) {
                *reinterpret_cast<float4 *>(Qt + e) = make_float4(qt[0], qt[1], qt[2], qt[3]);
                *reinterpret_cast<float4 *>(Kh + e) = make_float4(kh[0], kh[1], kh[2], kh[3]);
            }
        }
    }
    __syncthreads();
    if (FULL) {
        tri_form2(c.A, c.Bq, c.K, c.Q, c.G, DK);
    }
    if (FULL)
    // Tm = (I + Diag(beta) A)^-1 (unit lower triangular) by forward substitution: lane j of
    // wave 0 owns column j in registers (the loops are unrolled), so row i needs only row i
    // of A, read from LDS as float4s that every lane shares.  Entries above the diagonal
    // come out as (signed) zeros: their sums only see the column's zeros above the diagonal.
    {
        float *Al = lw, *Tl = lw + BC * BC, *bl = Tl + BC * BC;
        stage_rows(Al, c.A, BC, BC, BC, BC);
        if (tid < BC) bl[tid] = c.beta[tid];
        __syncthreads();
        if (tid < BC) {
            const int j = tid;
            float t[BC];
#pragma unroll
            for (int i = 0; i < BC; ++i) {
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                for (int u = 0; u + 4 <= i; u += 4) {
                    const float4 av = *reinterpret_cast<const float4 *>(Al + i * BC + u);
                    s0 = fmaf(av.x, t[u], s0);
                    s1 = fmaf(av.y, t[u + 1], s1);
                    s2 = fmaf(av.z, t[u + 2], s2);
                    s3 = fmaf(av.w, t[u + 3], s3);
                }
#pragma unroll
                for (int u = i & ~3; u < i; ++u) s0 = fmaf(Al[i * BC + u], t[u], s0);
                const float x = -bl[i] * ((s0 + s1) + (s2 + s3));
                t[i] = i == j ? 1.f : x;
            }
#pragma unroll
            for (int i = 0; i < BC; ++i) Tl[i * BC + j] = t[i];
        }
        __syncthreads();
        // Tm to the record, and Tm Diag(beta) for W = Tm Diag(beta) Kt and
        // Ut = Tm Diag(beta) V: the column scaling of one 64 x 64 matrix instead of scaled
        // copies of Kt and V
        float *__restrict__ TmB = c.TmB;
        for (int e4 = tid; e4 < BC * BC / 4; e4 += BT) {
            const float4 t = *reinterpret_cast<const float4 *>(Tl + 4 * e4);
            const int j = (4 * e4) % BC;
            *reinterpret_cast<float4 *>(c.Tm + 4 * e4) = t;
            *reinterpret_cast<float4 *>(TmB + 4 * e4) =
                make_float4(t.x * bl[j], t.y * bl[j + 1], t.z * bl[j + 2], t.w * bl[j + 3]);
        }
    }
    __syncthreads();
    if (FULL) {   // (the gradient kernel folds beta into its products instead)
        if (DK == DV) {   // one pass staging Tm Diag(beta) once for both
            gemm2_nn(c.W, c.Ut, DK, c.TmB, BC, c.Kt, c.V, DK, BC, DK, BC, tA, tB);
        } else {
            gemm<false, false>(c.W, DK, c.TmB, BC, c.Kt, DK, BC, DK, BC, 1.f, false, kNoMask, tA, tB);
            gemm<false, false>(c.Ut, DV, c.TmB, BC, c.V, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);
        }
    }
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
    c.Qt = s; s += mk;
    c.Kh = s; s += mk;
    c.A = s; s += mc;
    c.Bq = s; s += mc;
    c.Tm = s; s += mc;
    c.TmB = s; s += mv;   // (64 x 64 in use; sized as before)
    s += mk;
    c.W = s; s += mk;
    c.Ut = s; s += mv;
    c.beta = s; s += BC;
    c.eC = s; s += DK;
    *rest = s;
    return c;
}

// Per-chunk record written by bwd_prep and read by the two ordered passes.
struct Rec {
    float *Qt, *Kh, *W, *Ut, *Bq, *A, *Tm, *eC;
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
    r.A = p; p += (size_t)BC * BC;
    r.Tm = p; p += (size_t)BC * BC;
    r.eC = p;
    return r;
}

template <typename T>
__global__ __launch_bounds__(BT) void bwd_prep_kernel(KdaBwdArgs a) {
    // one panel area: the two panels of the products, and scratch of 2 kPanel rows elsewhere
    __shared__ __attribute__((aligned(16))) float panels[2 * kPanel][kPs];
    float(*tA)[kPs] = panels;
    float(*tB)[kPs] = panels + kPanel;
    float *rest;
    const ChunkMats c = carve(a.scratch + (size_t)blockIdx.x * a.scratch_floats, a.dk, a.dv, &rest);
    const int items = a.B * a.H * a.n_chunks;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int bh = it / a.n_chunks, n = it % a.n_chunks;
        // the matrices the ordered passes read are formed in place in the chunk's record
        const Rec r = rec_at(a, bh, n);
        ChunkMats cr = c;
        cr.Qt = r.Qt;
        cr.Kh = r.Kh;
        cr.W = r.W;
        cr.Ut = r.Ut;
        cr.Bq = r.Bq;
        cr.A = r.A;
        cr.Tm = r.Tm;
        cr.eC = r.eC;
        chunk_forward<T, true>(a, cr, bh, n, tA, tB);   // ends with a barrier
    }
}

// C[m][n] += scale * sum_k At[k*lda + m] B[k*ldb + n] (C = that sum when !acc), all in
// LDS, for N = 16, M a multiple of 16 and K = 64 or 128, on the fp32 matrix cores:
// the 16 x 16 output blocks go round the four waves, each a chain of K / 4 steps of
// v_mfma_f32_16x16x4_f32 (lane l supplies A[l%16][k + l/16] and B[k + l/16][l%16]) over
// two interleaved accumulators.
template <int K>
__device__ __forceinline__ void lds_mm_k(float *C, int ldc, const float *At, int lda, const float *B, int ldb, int M,
                                         float scale, bool acc) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, g = lane / 16, l16 = lane % 16;
    for (int rb = wave; rb < M / 16; rb += BT / 64) {
        f32x4_t c0 = zero4(), c1 = zero4();
        const float *a = At + g * lda + rb * 16 + l16;
        const float *b = B + g * ldb + l16;
#pragma unroll
        for (int k = 0; k < K; k += 8) {
            c0 = mma4(a[k * lda], b[k * ldb], c0);
            c1 = mma4(a[(k + 4) * lda], b[(k + 4) * ldb], c1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *p = C + (rb * 16 + 4 * g + i) * ldc + l16;
            const float x = scale * (c0[i] + c1[i]);
            *p = acc ? *p + x : x;
        }
    }
}
__device__ __forceinline__ void lds_mm(float *C, int ldc, const float *At, int lda, const float *B, int ldb, int M,
                                       int K, float scale, bool acc) {
    if (K == 128)
        lds_mm_k<128>(C, ldc, At, lda, B, ldb, M, scale, acc);
    else
        lds_mm_k<64>(C, ldc, At, lda, B, ldb, M, scale, acc);
}

// Copy n floats (a multiple of 4, 16-byte aligned) from global memory to registers, 4 per
// thread per slot, through a buffer resource: one lane offset for every slot, the slot in
// the scalar offset, and slots past n read zeros (range-checked), so no load sits under a
// branch and all of them stay in flight until the values are stored.
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <int SLOTS>
struct Pre {
    f32x4v r[SLOTS];
    __device__ __forceinline__ void load(const float *src, int n) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, n * 4, kBufWord3);
        const unsigned voff = 16u * threadIdx.x;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i)
            r[i] = __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 4096u * i, 0));
    }
    // element (r, c) of a row-major [n / cols][cols] matrix to dst[c * ldt + r]
    __device__ __forceinline__ void store_t(float *dst, int n, int cols, int ldt) const {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 4 * (threadIdx.x + BT * i);
            if (e < n) {
                const int row = e / cols, col = e % cols;
                dst[(col + 0) * ldt + row] = r[i].x;
                dst[(col + 1) * ldt + row] = r[i].y;
                dst[(col + 2) * ldt + row] = r[i].z;
                dst[(col + 3) * ldt + row] = r[i].w;
            }
        }
    }
    __device__ __forceinline__ void store(float *dst, int n) const {
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int e = 4 * (threadIdx.x + BT * i);
            if (e < n) *reinterpret_cast<f32x4v *>(dst + e) = r[i];
        }
    }
};
constexpr int SW = 16;                         // value columns per workgroup of the ordered passes
constexpr int kMatSlots = BC * 128 / (4 * BT); // float4 slots per thread for a 64 x 128 matrix
constexpr int kSqSlots = BC * BC / (4 * BT);   // for a 64 x 64 matrix

// Register prefetch of an ordered pass's small per-chunk operands: a [BC][SW] column slice
// of a row-major matrix (4 values per thread: row tid / 4, columns 4 (tid % 4) ..; rows at
// or past nr are read from row 0 and stored as zeros) and the chunk's DK decay factors.
// The loads carry no branch, so they stay in flight through the chunk's products.
template <typename T>
struct SlicePre {
    float v[4], e[4];
    int ok;
    __device__ __forceinline__ void load(const T *base, size_t row_stride, int nr, const float *eC, int DK) {
        const int r = threadIdx.x / 4;
        ok = r < nr;
        ld4(base + (size_t)(ok ? r : 0) * row_stride + 4 * (threadIdx.x % 4), v);
        ld4(eC + 4 * min((int)threadIdx.x, DK / 4 - 1), e);
    }
    __device__ __forceinline__ void store(float *slice, float *eCl, int DK) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) slice[4 * threadIdx.x + i] = ok ? v[i] : 0.f;
        if ((int)threadIdx.x < DK / 4)
#pragma unroll
            for (int i = 0; i < 4; ++i) eCl[4 * threadIdx.x + i] = e[i];
    }
};
static_assert(BC * SW == 4 * BT, "one 4-value piece of a column slice per thread");
static_assert(SW == 16, "the ordered passes' products are 16 columns wide");

// The ordered passes' workgroup index, regrouped so that the column blocks of one (batch,
// head) run on one XCD and read the chunk operands through its L2: workgroups are dealt to
// the 8 XCDs round robin, so workgroup i goes to XCD i % 8, and XCD x takes the logical
// blocks x * n / 8 .. (x + 1) * n / 8 - 1 (a bijection when n is a multiple of 8).
__device__ __forceinline__ int xcd_grouped_block() {
    const int i = blockIdx.x, n = gridDim.x;
    return n % 8 ? i : (i % 8) * (n / 8) + i / 8;
}

// The ordered passes share data between their threads through LDS only, so their barriers
// wait for LDS traffic alone (lds_barrier): the next chunk's register prefetch, issued a
// matrix at a time between the products, and the per-chunk state stores stay in flight.
//
// State at the start of every chunk: S_{n+1} = Diag(eC) S_n + Kh^T (Ut - W S_n), per SW value
// columns.  The state and the chunk's operands live in LDS; the next chunk's W and Kh are
// loaded into registers while the current one is computed.
// (L: this workgroup's logical index among the pass's B * H * DV / SW; lds: the LDS area)
__device__ void states_pass(const KdaBwdArgs &a, int L, float *lds) {
    float *S = lds, *U = S + 128 * SW, *Wt = U + BC * SW, *Khl = Wt + 128 * (BC + 1), *Utl = Khl + BC * 128,
          *eCl = Utl + BC * SW;
    const int DK = a.dk, DV = a.dv, nvs = DV / SW;
    const int bh = L / nvs, j0 = (L % nvs) * SW;
    for (int e = threadIdx.x; e < DK * SW; e += BT) S[e] = a.s0 ? a.s0[((size_t)bh * DK + e / SW) * DV + j0 + e % SW] : 0.f;
    Pre<kMatSlots> pw, pk;
    SlicePre<float> pu;
    {
        const Rec r = rec_at(a, bh, 0);
        pw.load(r.W, BC * DK);
        pk.load(r.Kh, BC * DK);
        pu.load(r.Ut + j0, DV, BC, r.eC, DK);
    }
    for (int n = 0; n < a.n_chunks; ++n) {
        lds_barrier();                         // the previous step is done with the LDS operands
        pw.store_t(Wt, BC * DK, DK, BC + 1);   // W^T, [DK][BC + 1]
        pk.store(Khl, BC * DK);
        pu.store(Utl, eCl, DK);
        float *Sn = a.states + ((size_t)bh * a.n_chunks + n) * DK * DV;
        for (int e = threadIdx.x; e < DK * SW; e += BT) Sn[(size_t)(e / SW) * DV + j0 + e % SW] = S[e];
        lds_barrier();
        // the next chunk's operands, each ahead of the product after which it is stored (the
        // last step reads its own chunk again, unused)
        const Rec r1 = rec_at(a, bh, min(n + 1, a.n_chunks - 1));
        pw.load(r1.W, BC * DK);
        pu.load(r1.Ut + j0, DV, BC, r1.eC, DK);
        for (int e = threadIdx.x; e < BC * SW; e += BT) U[e] = Utl[e];
        lds_barrier();
        lds_mm(U, SW, Wt, BC + 1, S, SW, BC, DK, -1.f, true);            // U = Ut - W S
        lds_barrier();
        pk.load(r1.Kh, BC * DK);
        for (int e = threadIdx.x; e < DK * SW; e += BT) S[e] *= eCl[e / SW];
        lds_barrier();
        lds_mm(S, SW, Khl, DK, U, SW, DK, BC, 1.f, true);                // S += Kh^T U
    }
}

// Reverse pass: dS' of every chunk (the gradient of the state after it) and dS0, per SW
// value columns, with the same LDS layout and register prefetch.
template <typename T>
__device__ void reverse_pass(const KdaBwdArgs &a, int L, float *lds) {
    float *dS = lds, *dSn = dS + 128 * SW, *dU = dSn + 128 * SW, *dO = dU + BC * SW, *Bql = dO + BC * SW,
          *Kht = Bql + BC * BC, *Qtl = Kht + 128 * (BC + 1), *Wl = Qtl + BC * 128, *eCl = Wl + BC * 128;
    const int DK = a.dk, DV = a.dv, H = a.H, nvs = DV / SW;
    const int bh = L / nvs, j0 = (L % nvs) * SW, b = bh / H, h = bh % H;
    const T *go = static_cast<const T *>(a.dO);
    for (int e = threadIdx.x; e < DK * SW; e += BT)
        dS[e] = a.dsT ? a.dsT[((size_t)bh * DK + e / SW) * DV + j0 + e % SW] : 0.f;
    const T *go_bh = go + ((size_t)b * a.T * H + h) * DV + j0;   // dO of this (batch, head), columns j0 ..
    const size_t chunk_rows = (size_t)BC * H * DV;                  // its offset per chunk
    Pre<kSqSlots> pb;
    Pre<kMatSlots> pk, pq, pw;
    SlicePre<T> po;
    {
        const int n = a.n_chunks - 1;
        const Rec r = rec_at(a, bh, n);
        pb.load(r.Bq, BC * BC);
        pk.load(r.Kh, BC * DK);
        pq.load(r.Qt, BC * DK);
        pw.load(r.W, BC * DK);
        po.load(go_bh + n * chunk_rows, (size_t)H * DV, min(BC, a.T - n * BC), r.eC, DK);
    }
    for (int n = a.n_chunks - 1; n >= 0; --n) {
        lds_barrier();
        pb.store(Bql, BC * BC);
        pk.store_t(Kht, BC * DK, DK, BC + 1);  // Kh^T, [DK][BC + 1]
        pq.store(Qtl, BC * DK);
        pw.store(Wl, BC * DK);
        po.store(dO, eCl, DK);
        float *dSp = a.dstates + ((size_t)bh * a.n_chunks + n) * DK * DV;
        for (int e = threadIdx.x; e < DK * SW; e += BT) dSp[(size_t)(e / SW) * DV + j0 + e % SW] = dS[e];
        lds_barrier();
        // the next chunk's operands, one matrix ahead of each product so that the loads go
        // through the memory pipeline under the products (at n = 0 chunk 0 is read again,
        // unused); the barriers between the products wait for LDS only, leaving them in flight
        const int np = max(n - 1, 0);
        const Rec r1 = rec_at(a, bh, np);
        pb.load(r1.Bq, BC * BC);
        po.load(go_bh + np * chunk_rows, (size_t)H * DV, min(BC, a.T - np * BC), r1.eC, DK);
        lds_mm(dU, SW, Bql, BC, dO, SW, BC, BC, 1.f, false);            // dU = Bq^T dO
        lds_barrier();
        pk.load(r1.Kh, BC * DK);
        lds_mm(dU, SW, Kht, BC + 1, dS, SW, BC, DK, 1.f, true);         //    + Kh dS'
        for (int e = threadIdx.x; e < DK * SW; e += BT) dSn[e] = eCl[e / SW] * dS[e];
        lds_barrier();
        pq.load(r1.Qt, BC * DK);
        lds_mm(dSn, SW, Qtl, DK, dO, SW, DK, BC, 1.f, true);            // + Qt^T dO
        lds_barrier();
        pw.load(r1.W, BC * DK);
        lds_mm(dSn, SW, Wl, DK, dU, SW, DK, BC, -1.f, true);            // - W^T dU
        lds_barrier();
        for (int e = threadIdx.x; e < DK * SW; e += BT) dS[e] = dSn[e];
    }
    __syncthreads();
    if (a.ds0)
        for (int e = threadIdx.x; e < DK * SW; e += BT) a.ds0[((size_t)bh * DK + e / SW) * DV + j0 + e % SW] = dS[e];
}

// The two ordered passes need only the per-chunk records, not each other's results, so they
// run side by side in one launch: workgroups 0 .. n_states-1 (logical) compute the states,
// the rest the reverse pass, each half over whole XCDs.
constexpr int kStatesLds = 128 * SW + 2 * BC * SW + 128 * (BC + 1) + BC * 128 + 128;
constexpr int kReverseLds = 2 * 128 * SW + 2 * BC * SW + BC * BC + 128 * (BC + 1) + 2 * BC * 128 + 128;
constexpr int kOrderedLds = kStatesLds > kReverseLds ? kStatesLds : kReverseLds;
static_assert(kOrderedLds * 4 <= 160 * 1024, "the ordered passes' LDS fits a CU");
template <typename T>
__global__ __launch_bounds__(BT) void bwd_ordered_kernel(KdaBwdArgs a, int n_states) {
    __shared__ __attribute__((aligned(16))) float lds[kOrderedLds];
    const int L = xcd_grouped_block();
    if (L < n_states)
        states_pass(a, L, lds);
    else
        reverse_pass<T>(a, L - n_states, lds);
}

// Gradients of one chunk's tokens.
template <typename T>
__global__ __launch_bounds__(BT, 2) void bwd_intra_kernel(KdaBwdArgs a) {
    // one panel area: the two panels of the products, and scratch of 2 kPanel rows elsewhere
    __shared__ __attribute__((aligned(16))) float panels[2 * kPanel][kPs];
    float(*tA)[kPs] = panels;
    float(*tB)[kPs] = panels + kPanel;
    const int DK = a.dk, DV = a.dv, H = a.H, tid = threadIdx.x;
    float *s;
    const ChunkMats base = carve(a.scratch + (size_t)blockIdx.x * a.scratch_floats, DK, DV, &s);
    const size_t mk = (size_t)BC * DK, mv = (size_t)BC * DV, mc = (size_t)BC * BC;
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
    float *dKx = s; s += mk;   // R(dA, K): the row side of A
    float *dKy = s; s += mk;   // C(dA, K) + C(dBq, Q): the column side of A and Bq
    float *dQi = dW;           // R(dBq, K), once dW is spent
    T *gq = static_cast<T *>(a.dq), *gk = static_cast<T *>(a.dk_out), *gv = static_cast<T *>(a.dv_out);
    T *ga = static_cast<T *>(a.dalpha), *gb = static_cast<T *>(a.dbeta);
    const T *go = static_cast<const T *>(a.dO), *al = static_cast<const T *>(a.alpha);
    const int items = a.B * H * a.n_chunks;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int bh = it / a.n_chunks, n = it % a.n_chunks, b = bh / H, h = bh % H;
        const int t0 = n * BC, nr = min(BC, a.T - t0);
        auto tok = [&](int r) { return ((size_t)b * a.T + t0 + r) * H + h; };
        // the record's matrices (Qt, Kh, A, Bq, Tm, W, Ut, exp(gC)) plus the rest rebuilt;
        // U = Ut - W S is formed in place of the record's Ut, which nothing reads any more
        const Rec rc = rec_at(a, bh, n);
        ChunkMats c = base;
        c.Qt = rc.Qt;
        c.Kh = rc.Kh;
        c.W = rc.W;
        c.Ut = rc.Ut;
        c.Bq = rc.Bq;
        c.A = rc.A;
        c.Tm = rc.Tm;
        c.eC = rc.eC;
        float *U = c.Ut;
        chunk_forward<T, false>(a, c, bh, n, tA, tB);
        const float *Sn = a.states + ((size_t)bh * a.n_chunks + n) * DK * DV;
        const float *dSp = a.dstates + ((size_t)bh * a.n_chunks + n) * DK * DV;
        stage_rows(dO, go + tok(0) * DV, (size_t)H * DV, BC, DV, nr);
        __syncthreads();
        gemm<false, false>(U, DV, c.W, DK, Sn, DV, BC, DV, DK, -1.f, true, kNoMask, tA, tB);        // U = Ut - W S
        gemm<true, false>(dU, DV, c.Bq, BC, dO, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);       // dU = Bq^T dO
        gemm<false, false>(dU, DV, c.Kh, DK, dSp, DV, BC, DV, DK, 1.f, true, kNoMask, tA, tB);      //    + Kh dS'
        gemm<false, true>(dBq, BC, dO, DV, U, DV, BC, BC, DV, 1.f, false, kLower, tA, tB);          // dBq
        gemm2_nt(dQt, 1.f, dO, dW, -1.f, dU, DV, Sn, DV, DK, BC, DK, DV, tA, tB);                   // dQt = dO S^T, dW = -dU S^T
        gemm<false, true>(dKh, DK, U, DV, dSp, DV, BC, DK, DV, 1.f, false, kNoMask, tA, tB);        // dKh = U dS'^T
        // dTm = dU X^T + dW Y^T = (dU V^T + dW Kt^T) Diag(beta), and Tm^T dTm takes the same column
        // scaling: the products run on V and Kt, and beta scales the columns of Tm^T dTm
        gemm<false, true>(dTm, BC, dU, DV, c.V, DV, BC, BC, DV, 1.f, false, kNoMask, tA, tB);       // dU V^T
        gemm<false, true>(dTm, BC, dW, DK, c.Kt, DK, BC, BC, DK, 1.f, true, kNoMask, tA, tB);       //  + dW Kt^T
        gemm<true, false>(P, BC, c.Tm, BC, dTm, BC, BC, BC, BC, 1.f, false, kNoMask, tA, tB);       // Tm^T (...)
        for (int e = tid; e < BC * BC; e += BT) P[e] *= c.beta[e % BC];                             //  Diag(beta)
        __syncthreads();
        gemm<false, true>(dM, BC, P, BC, c.Tm, BC, BC, BC, BC, -1.f, false, kNoMask, tA, tB);       // dM
        gemm<true, false>(dX, DV, c.Tm, BC, dU, DV, BC, DV, BC, 1.f, false, kNoMask, tA, tB);       // dX = Tm^T dU
        gemm<true, false>(dY, DK, c.Tm, BC, dW, DK, BC, DK, BC, 1.f, false, kNoMask, tA, tB);       // dY = Tm^T dW
        // dA = strict_lower(Diag(beta) dM), in P
        for (int e = tid; e < BC * BC; e += BT) {
            const int r = e / BC, s2 = e % BC;
            P[e] = s2 < r ? c.beta[r] * dM[e] : 0.f;
        }
        __syncthreads();
        tri_rows2(dKx, P, dQi, dBq, c.K, c.G, DK);      // R(dA, K), R(dBq, K)
        tri_cols2(dKy, P, c.K, dBq, c.Q, c.G, DK);      // C(dA, K) + C(dBq, Q)
        // the panel area as scratch from here on: dG [BC][DK], alpha [BC][DK], partial sums
        float *lw = &tA[0][0];
        float *dGl = lw, *alpha_l = lw + BC * DK, *part = lw + 2 * BC * DK;   // part: 4 BC + 4 DK + 2 DK floats
        static_assert(2 * BC * 128 + 4 * BC + 6 * 128 <= 2 * kPanel * kPs, "the tail's LDS fits the panel area");
        stage_rows(alpha_l, al + tok(0) * DK, (size_t)H * DK, BC, DK, nr);
        // dbeta: four threads per row, each a quarter of the three row sums
        {
            // fixed trip counts with masked terms (indices clamped in range), so every load of
            // a loop is issued before the first sum needs one
            const int r = tid / 4, q = tid % 4, nv = DV / 16, nk = DK / 16;   // nv, nk: 4 or 8
            float db = 0.f;
#pragma unroll 8
            for (int i = 0; i < 16; ++i) {
                const int s2 = 16 * q + i;
                const float x = dM[r * BC + s2] * c.A[r * BC + s2];
                db += s2 < r ? x : 0.f;
            }
#pragma unroll 4
            for (int i = 0; i < 8; ++i) {
                const int j4 = q * nv + min(i, nv - 1);
                const float4 x = *reinterpret_cast<const float4 *>(dX + r * DV + 4 * j4);
                const float4 w = *reinterpret_cast<const float4 *>(c.V + r * DV + 4 * j4);
                const float d = x.x * w.x + x.y * w.y + x.z * w.z + x.w * w.w;
                db += i < nv ? d : 0.f;
            }
#pragma unroll 4
            for (int i = 0; i < 8; ++i) {
                const int c4 = q * nk + min(i, nk - 1);
                const float4 x = *reinterpret_cast<const float4 *>(dY + r * DK + 4 * c4);
                const float4 w = *reinterpret_cast<const float4 *>(c.Kt + r * DK + 4 * c4);
                const float d = x.x * w.x + x.y * w.y + x.z * w.z + x.w * w.w;
                db += i < nk ? d : 0.f;
            }
            part[4 * r + q] = db;
        }
        // dv, dq, dk and dG (into LDS)
        for (int e4 = tid; e4 < BC * DV / 4; e4 += BT) {
            const int e = 4 * e4, r = e / DV;
            if (r < nr) {
                const float4 x = *reinterpret_cast<const float4 *>(dX + e);
                const float bb = c.beta[r];
                T *d = gv + tok(r) * DV + e % DV;
                st(d, bb * x.x);
                st(d + 1, bb * x.y);
                st(d + 2, bb * x.z);
                st(d + 3, bb * x.w);
            }
        }
        for (int e4 = tid; e4 < BC * DK / 4; e4 += BT) {
            const int e = 4 * e4, r = e / DK, ch = e % DK;
            const float bb = c.beta[r];
            float g4[4], gc[4], q1[4], qi[4], y1[4], kx[4], ky[4], h1[4], qr[4], kr[4];
            ld4(c.G + e, g4);
            ld4(c.G + (BC - 1) * DK + ch, gc);   // gC: rows past the end repeat the last valid row's G
            ld4(dQt + e, q1);
            ld4(dQi + e, qi);
            ld4(dY + e, y1);
            ld4(dKx + e, kx);
            ld4(dKy + e, ky);
            ld4(dKh + e, h1);
            ld4(c.Q + e, qr);
            ld4(c.K + e, kr);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gm = exp2f(g4[i]);
                const float dq = gm * q1[i] + qi[i];
                const float dkx = gm * bb * y1[i] + kx[i];
                const float dkh = exp2f(gc[i] - g4[i]) * h1[i];
                if (r < nr) {
                    st(gq + tok(r) * DK + ch + i, dq);
                    st(gk + tok(r) * DK + ch + i, dkx + ky[i] + dkh);
                }
                dGl[e + i] = qr[i] * dq + kr[i] * (dkx - ky[i] - dkh);
            }
        }
        // the last row's extra terms: colsum(dKh * Kh) over the rows (four row groups of
        // sixteen, four channels per thread) and exp(gC) rowsum(dS' * S) over the value columns
        float *colp = part + 4 * BC, *sdsp = part + 4 * BC + 4 * DK;
        for (int w = tid; w < 4 * DK / 4; w += BT) {
            const int c4 = w % (DK / 4), rg = w / (DK / 4);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = 16 * rg; r < 16 * rg + 16; ++r) {
                const float4 x = *reinterpret_cast<const float4 *>(dKh + r * DK + 4 * c4);
                const float4 y = *reinterpret_cast<const float4 *>(c.Kh + r * DK + 4 * c4);
                acc.x += x.x * y.x;
                acc.y += x.y * y.y;
                acc.z += x.z * y.z;
                acc.w += x.w * y.w;
            }
            *reinterpret_cast<float4 *>(colp + rg * DK + 4 * c4) = acc;
        }
        for (int w = tid; w < 2 * DK; w += BT) {
            const int ch = w / 2, half = w % 2;
            float acc = 0.f;
            for (int j4 = half * DV / 8; j4 < (half + 1) * DV / 8; ++j4) {
                const float4 x = *reinterpret_cast<const float4 *>(dSp + (size_t)ch * DV + 4 * j4);
                const float4 y = *reinterpret_cast<const float4 *>(Sn + (size_t)ch * DV + 4 * j4);
                acc += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
            }
            sdsp[w] = acc;
        }
        __syncthreads();
        if (tid < nr) st(gb + tok(tid), part[4 * tid] + part[4 * tid + 1] + part[4 * tid + 2] + part[4 * tid + 3]);
        // the chunk's last row is its last valid token: rows past the end contribute nothing;
        // then the reverse cumulative sum down the rows gives dlog alpha
        for (int ch = tid; ch < DK; ch += BT) {
            float extra = 0.f;
            for (int rg = 0; rg < 4; ++rg) extra += colp[rg * DK + ch];
            const int last = nr - 1;
            dGl[last * DK + ch] += extra + c.eC[ch] * (sdsp[2 * ch] + sdsp[2 * ch + 1]);
            float run = 0.f;
            for (int r = last; r >= 0; --r) {
                run += dGl[r * DK + ch];
                st(ga + tok(r) * DK + ch, run / alpha_l[r * DK + ch]);
            }
        }
        __syncthreads();
    }
}

}  // namespace

size_t kda_bwd_scratch_floats(int dk, int dv) {
    const size_t mk = (size_t)BC * dk, mv = (size_t)BC * dv, mc = (size_t)BC * BC;
    // ChunkMats + the intra kernel's temporaries (the largest user)
    const size_t chunk = 8 * mk + 4 * mv + 3 * mc + BC + dk;
    const size_t intra = 3 * mv + 4 * mc + 6 * mk;
    return chunk + intra + 64;
}

size_t kda_bwd_rec_floats(int dk, int dv) { return 3 * (size_t)BC * dk + (size_t)BC * dv + 3 * (size_t)BC * BC + dk; }

hipError_t launch_kda_backward(KdaBwdArgs a, bool bf16, hipStream_t stream) {
    if (a.B * a.H == 0) return hipSuccess;
    const int items = a.B * a.H * a.n_chunks;
    const int g = items < kBwdBlocks ? items : kBwdBlocks;
    const int ordered = a.B * a.H * (a.dv / SW);
    if (bf16) {
        hipLaunchKernelGGL(bwd_prep_kernel<bf16_t>, dim3(g), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_ordered_kernel<bf16_t>, dim3(2 * ordered), dim3(BT), 0, stream, a, ordered);
        hipLaunchKernelGGL(bwd_intra_kernel<bf16_t>, dim3(g), dim3(BT), 0, stream, a);
    } else {
        hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(g), dim3(BT), 0, stream, a);
        hipLaunchKernelGGL(bwd_ordered_kernel<float>, dim3(2 * ordered), dim3(BT), 0, stream, a, ordered);
        hipLaunchKernelGGL(bwd_intra_kernel<float>, dim3(g), dim3(BT), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kdaconv
