// Chunked Kimi Delta Attention forward for gfx950: intra-chunk UT/WY kernel
// and the sequential inter-chunk state pass.
//
// Per (batch, head), with chunk tokens r = 0..63, key channel c and
// G_r = sum_{u<=r} log2 alpha_u (per channel), the gated delta rule
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t                                      (Chimera, method step (5))
// regroups chunkwise into
//   A  = strict-lower( sum_c k_r k_s 2^(G_r - G_s) ),   Bq = lower( sum_c q_r k_s 2^(G_r - G_s) )
//   Tm = (I + Diag(beta) A)^-1
//   W  = Tm Diag(beta) (2^G * K),   Ut = Tm Diag(beta) V,   Qt = 2^G * Q
//   Kh = 2^(G_63 - G) * K,          Gam = 2^(G_63)
// and, walking the chunks in order with the state S (dk x dv, fp32):
//   U = Ut - W S;   O = Qt S + Bq U;   S <- Diag(Gam) S + Kh^T U.
//
// Kernel 1 (kda_intra_kernel: persistent, one 8-wave workgroup per CU, each
// chunk fully independent) forms W, Qt, Kh, Bq^T, Ut and Gam and writes them
// to the workspace in the exact register-fragment order kernel 2 consumes.
// The next chunk's inputs are loaded into registers while the current chunk
// is transformed.
// Kernel 2 (kda_state_kernel: one 8-wave workgroup per (batch, head,
// 16-column slice of dv)) keeps its state slice in the registers of one
// recurrence wave and feeds it to the matrix cores without any reshuffle;
// four loader waves stage the chunk operands in an LDS ring, two output waves
// and a store wave form and write o from the state handed over each step.
//
// Decay factorisation: 2^(G_r - G_s) for s <= r is split around the midpoint
// m(R) = 16R + 8 of the 16-row sub-block R of row r:
//   Kr_r = k_r 2^(G_r - G_m(R)),  Qr_r = q_r 2^(G_r - G_m(R)),  Kb_s = k_s 2^(G_m(S) - G_s)
//   sub-block (R, S <= R):  A_RS = Kr_R Diag(2^(G_m(R) - G_m(S))) Kb_S^T  (same for Bq with Qr).
// Every factor is <= 1 except inside one sub-block, where it spans at most 8
// tokens; off-diagonal factors never overflow.
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace kdaconv {
namespace {

constexpr int C = kChunk;          // 64 tokens per chunk
constexpr int K1_THREADS = 512;    // 8 waves

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
// 4 DK/16 values a kernel-2 lane group g needs are contiguous, 2 per lane.
template <int DK> __device__ __forceinline__ int gam_pos(int c) {
    return ((c >> 2) & 3) * (DK / 4) + 4 * (c >> 4) + (c & 3);
}

// ---- raw 8-element rows (register prefetch without conversion) --------------
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16_t *p) { u = *reinterpret_cast<const uint4 *>(p); }
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
    __device__ __forceinline__ void get(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};
template <typename T> struct Raw4;
template <> struct Raw4<bf16_t> {
    uint2 u;
    __device__ __forceinline__ void load(const bf16_t *p) { u = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = i < 2 ? u.x : u.y;
        return (i & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};
template <> struct Raw4<float> {
    float4 a;
    __device__ __forceinline__ void load(const float *p) { a = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ float get(int i) const { return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : a.w; }
};

// ---- kernel 1 shared-memory plan --------------------------------------------------
template <typename T, int DK, int DV>
struct K1Smem {
    static constexpr int NPART = K1_THREADS / DK;     // threads per channel in the table loop
    static constexpr int KP = 16 / (int)sizeof(T);
    static constexpr int KS = DK + KP;                // row stride of Kr, Qr, Kb
    static constexpr int RKS = 2 * (DK + 8 / (int)sizeof(T));  // row-pair stride of RHS_K
    static constexpr int RVS = 2 * (DV + 8 / (int)sizeof(T));  // row-pair stride of RHS_V
    static constexpr int LS = 64 + 4;                 // fp32 64x64 stride (Lm, Tm32)
    static constexpr int TS = 64 + KP;                // T 64x64 stride (Tm16)
    static constexpr int SC = 17;                     // 16x16 fp32 scratch stride

    static constexpr int GS = DK + 4;                 // fp32 row stride of G
    static constexpr size_t SZ_G = (size_t)C * GS * 4;
    static constexpr size_t SZ_LM = (size_t)C * LS * 4;
    static constexpr size_t SZ_K = (size_t)C * KS * sizeof(T);
    static constexpr size_t SZ_SCR = 8 * 16 * SC * 4;

    static constexpr size_t X1 = 0;   // G (P0-P1) | Lm + Tm32 (P2-P3)
    static constexpr size_t X1_SZ = round_up(SZ_G > 2 * SZ_LM ? SZ_G : 2 * SZ_LM, 16);
    static constexpr size_t X2 = X1 + X1_SZ;   // Kr + Kb (P1-P2, Kb until exported) | scratch (P3, at Kr)
    static constexpr size_t X2_SZ = round_up(2 * SZ_K > SZ_SCR ? 2 * SZ_K : SZ_SCR, 16);
    static constexpr size_t X3 = X2 + X2_SZ;   // Tm16 (P3-P5)
    static constexpr size_t Q = X3 + round_up((size_t)C * TS * sizeof(T), 16);   // Qr (P1-P2)
    static constexpr size_t RK = Q + round_up(SZ_K, 16);            // RHS_K row pairs (P1-P5)
    static constexpr size_t RV = RK + round_up((size_t)32 * RKS * sizeof(T), 16);
    static constexpr size_t TB = RV + round_up((size_t)32 * RVS * sizeof(T), 16);
    // tables (fp32): Pm[4][DK], Kh[4][DK], Fp[6][DK], beta[64]
    static constexpr size_t TB_PM = TB;
    static constexpr size_t TB_KH = TB_PM + 4 * DK * 4;
    static constexpr size_t TB_FP = TB_KH + 4 * DK * 4;
    static constexpr size_t TB_BETA = TB_FP + 6 * DK * 4;
    static constexpr size_t BYTES = round_up(TB_BETA + 64 * 4, 16);
};

__device__ __forceinline__ int fp_index(int R, int S) { return R * (R - 1) / 2 + S; }

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each 16-lane row (zeros shifted in), then lane 15 of rows 0 and 2
// into rows 1 and 3, then lane 31 into rows 2 and 3 (DPP row broadcasts).
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, BOUND));
}
// N independent scans, interleaved step by step (each DPP read then finds
// its source written N instructions earlier).
template <int N>
__device__ __forceinline__ void wave_inclusive_sums(float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x111, 0xf, true>(x[i]);   // row_shr:1
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x112, 0xf, true>(x[i]);   // row_shr:2
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x114, 0xf, true>(x[i]);   // row_shr:4
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x118, 0xf, true>(x[i]);   // row_shr:8
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x142, 0xa, false>(x[i]);  // row_bcast:15 -> rows 1, 3
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp_f<0x143, 0xc, false>(x[i]);  // row_bcast:31 -> rows 2, 3
}

// Hardware base-2 exponent and logarithm (v_exp_f32, v_log_f32, about 1 ulp).
// Results below the smallest normal flush to zero, which only affects decay
// factors far below any term they are added to; alpha is a positive normal
// number or exactly 1 (log2 = 0).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16x16x16 fp32 product X*Y with X, Y row-major in LDS; lane holds rows 4g+i of column col.
__device__ __forceinline__ f32x4_t mm16(const float *X, int ldx, const float *Y, int ldy, int col,
                                        int g, f32x4_t acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mma4(X[col * ldx + 4 * j + g], Y[(4 * j + g) * ldy + col], acc);
    return acc;
}

// Per-thread register prefetch of one chunk's inputs: rows 2rp, 2rp+1 of 8
// channels of alpha, k, q (key side) and of v (value side), plus beta.
template <typename T>
struct Prefetch {
    Raw8<T> a[2];         // alpha: row (lane) of the wave's channel slice, NA used
    Raw8<T> k[2], q[2], v[2];
    T beta;   // raw: converted where it is used, so the load is not waited for at issue
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(K1_THREADS) void kda_intra_kernel(KdaArgs a) {
    using SM = K1Smem<T, DK, DV>;
    using WL = Ws<T, DK, DV>;
    using F = Frag<T>;
    static_assert(SM::BYTES <= 160 * 1024, "LDS plan exceeds 160 KB");
    constexpr int NCGK = DK / 8, NCGV = DV / 8;   // 8-channel groups
    constexpr int CPW = DK / 8, NA = CPW / 8;      // P0: alpha channels per wave, 8-element loads per lane
    static_assert(K1_THREADS == 512 && C == 64 && NA >= 1 && NA <= 2, "P0 maps chunk rows to the 64 lanes of 8 waves");
    constexpr int NKS = DK / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, col = l & 15, g = l >> 4;
    // items: (chunk gc over all sequences, head h), chunk-major: item = gc * H + h
    const int total = seq_chk0(a, a.B);
    const int n_items = a.H * total;
    // an item's chunk: head, chunk index over all sequences, first token, valid rows
    struct Loc {
        int h, gc, t0, nr;
    };
    auto locate = [&](int it) {
        Loc L;
        L.h = it % a.H;
        L.gc = it / a.H;
        if (a.varlen) {
            const int sq = seq_of_chunk(a, L.gc);
            L.t0 = a.tok0[sq] + (L.gc - a.chk0[sq]) * C;
            L.nr = min(C, a.tok0[sq + 1] - L.t0);
        } else {
            const int sq = L.gc / a.n_chunks, n = L.gc - sq * a.n_chunks;
            L.t0 = sq * a.T + n * C;
            L.nr = min(C, a.T - n * C);
        }
        return L;
    };

    float *Gs = reinterpret_cast<float *>(smem + SM::X1);   // G, P0-P1 (Lm and Tm32 from P2 on)
    float *Lm = reinterpret_cast<float *>(smem + SM::X1);
    float *Tm32 = reinterpret_cast<float *>(smem + SM::X1 + SM::SZ_LM);
    T *Kr = reinterpret_cast<T *>(smem + SM::X2);
    T *Kb = reinterpret_cast<T *>(smem + SM::X2 + SM::SZ_K);
    float *Scr = reinterpret_cast<float *>(smem + SM::X2);
    T *Tm16 = reinterpret_cast<T *>(smem + SM::X3);
    T *Qr = reinterpret_cast<T *>(smem + SM::Q);
    T *RK = reinterpret_cast<T *>(smem + SM::RK);
    T *RV = reinterpret_cast<T *>(smem + SM::RV);
    float *Pm = reinterpret_cast<float *>(smem + SM::TB_PM);
    float *Kh = reinterpret_cast<float *>(smem + SM::TB_KH);
    float *Fp = reinterpret_cast<float *>(smem + SM::TB_FP);
    float *Bt = reinterpret_cast<float *>(smem + SM::TB_BETA);

    const T *q_in = static_cast<const T *>(a.q);
    const T *k_in = static_cast<const T *>(a.k);
    const T *v_in = static_cast<const T *>(a.v);
    const T *a_in = static_cast<const T *>(a.alpha);
    const T *b_in = static_cast<const T *>(a.beta);

    // thread roles of the elementwise phases
    const bool key_task = tid < 32 * NCGK, val_task = tid < 32 * NCGV;
    const int krp = tid / NCGK, kc0 = 8 * (tid % NCGK);
    const int vrp = tid / NCGV, vc0 = 8 * (tid % NCGV);

    // The next chunk's inputs are loaded into the prefetch registers part by
    // part, each as soon as the current chunk has consumed that part, so the
    // loads drain through the memory pipeline under the compute of P1-P3.
    constexpr int LD_A = 1, LD_KQ = 2, LD_V = 4;   // alpha and beta | k and q | v
    auto load_inputs = [&](const Loc &L, Prefetch<T> &pf, int parts) {
        const int h = L.h, t0 = L.t0, nr = L.nr;
        // Rows past the end of the sequence re-read the last row (in bounds) and
        // are masked where they are used: the loads never depend on the data
        // and no register is cleared behind a store still in flight.
        if (parts & LD_A) {
            const int r = min(l, nr - 1);
            const size_t off = ((size_t)(t0 + r) * a.H + h) * DK + CPW * wv;
#pragma unroll
            for (int j = 0; j < NA; ++j) pf.a[j].load(a_in + off + 8 * j);
            if (tid < C) pf.beta = b_in[(size_t)(t0 + min(tid, nr - 1)) * a.H + h];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if ((parts & LD_KQ) && key_task) {
                const int r = min(2 * krp + e, nr - 1);
                const size_t off = ((size_t)(t0 + r) * a.H + h) * DK + kc0;
                pf.k[e].load(k_in + off);
                pf.q[e].load(q_in + off);
            }
            if ((parts & LD_V) && val_task) {
                const int rv = min(2 * vrp + e, nr - 1);
                pf.v[e].load(v_in + ((size_t)(t0 + rv) * a.H + h) * DV + vc0);
            }
        }
    };

    Prefetch<T> pf;
    int item = blockIdx.x;
    Loc nxt{0, 0, 0, 0};   // the chunk whose inputs are in the prefetch registers
    if (item < n_items) {
        nxt = locate(item);
        load_inputs(nxt, pf, LD_A | LD_KQ | LD_V);
    }
    // Enter the loop with the first prefetch retired, as every later iteration
    // is (see P5): the loop's waits then never cover the stores still in flight.
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)

#pragma unroll 1
    for (; item < n_items; item += gridDim.x) {
        const Loc cur = nxt;
        const int nr = cur.nr;   // valid rows in this chunk
        const bool more = item + (int)gridDim.x < n_items;
        if (more) nxt = locate(item + gridDim.x);
        char *wsb = static_cast<char *>(a.ws) + ((size_t)cur.h * total + cur.gc) * WL::BYTES;
        T *ws = reinterpret_cast<T *>(wsb);
        float *ws_gam = reinterpret_cast<float *>(wsb + WL::GAM_BYTE);

        // ---- P0: G = cumsum(log2 alpha) over the chunk ------------------------------
        // Lane l of wave w holds row l of channels CPW*w .. CPW*w + CPW-1, so the
        // scan over the chunk's rows runs across the lanes of one wave (DPP
        // shifts inside 16-lane rows, then row broadcasts) with no barrier.
        {
            float x[CPW];
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                float v[8];
                pf.a[j].get(v);
#pragma unroll
                for (int i = 0; i < 8; ++i) x[8 * j + i] = l < nr ? hw_log2(v[i]) : 0.f;
            }
            wave_inclusive_sums<CPW>(x);
            float *d = Gs + l * SM::GS + CPW * wv;
#pragma unroll
            for (int i = 0; i < CPW; i += 4) *reinterpret_cast<float4 *>(d + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
        }
        if (tid < C) Bt[tid] = tid < nr ? (float)pf.beta : 0.f;
        lds_barrier();
        if (more) load_inputs(nxt, pf, LD_A);
        auto Grow = [&](int R) { return Gs + (R < 4 ? 16 * R + 8 : C - 1) * SM::GS; };   // R = 4: the last row
        {
            // 15 per-channel factors for the later phases: Pm[4], Kh[4], Fp[6], Gam
            // (P1 computes its own Pm values: the tables are read from P2 on).
            // The five G rows are read once, up front.
            const int c = tid % DK, part = tid / DK;
            float gv[5];
#pragma unroll
            for (int R = 0; R < 5; ++R) gv[R] = Grow(R)[c];
#pragma unroll
            for (int j = 0; j < (15 + SM::NPART - 1) / SM::NPART; ++j) {
                const int e = part + SM::NPART * j;
                if (e < 4) {
                    Pm[e * DK + c] = hw_exp2(gv[e & 3]);
                } else if (e < 8) {
                    Kh[(e - 4) * DK + c] = hw_exp2(gv[4] - gv[e & 3]);
                } else if (e < 14) {
                    const int f = e - 8;
                    const int R = f < 1 ? 1 : (f < 3 ? 2 : 3);
                    const int S = f - fp_index(R, 0);
                    Fp[f * DK + c] = hw_exp2(gv[R] - gv[S]);
                } else if (e == 14) {
                    ws_gam[gam_pos<DK>(c)] = hw_exp2(gv[4]);
                }
            }
        }

        // ---- P1: elementwise operands ----------------------------------------------
        if (key_task) {
            const int s0 = 2 * krp, R = s0 >> 4;
            float gm[8], pm[8];   // G at the block midpoint 16R+8, and 2^G there
            {
                const float4 m0 = *reinterpret_cast<const float4 *>(Grow(R) + kc0);
                const float4 m1 = *reinterpret_cast<const float4 *>(Grow(R) + kc0 + 4);
                gm[0] = m0.x; gm[1] = m0.y; gm[2] = m0.z; gm[3] = m0.w;
                gm[4] = m1.x; gm[5] = m1.y; gm[6] = m1.z; gm[7] = m1.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) pm[i] = hw_exp2(gm[i]);
            float rhs[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = s0 + e;
                float kx[8], qx[8];
                pf.k[e].get(kx);
                pf.q[e].get(qx);
#pragma unroll
                for (int i = 0; i < 8; ++i) {   // rows past the stream end are zero
                    kx[i] = r < nr ? kx[i] : 0.f;
                    qx[i] = r < nr ? qx[i] : 0.f;
                }
                const float br = Bt[r];
                float kr[8], qr[8], kb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = Gs[r * SM::GS + kc0 + i] - gm[i];
                    const float e1 = hw_exp2(d), e2 = hw_exp2(-d);
                    kr[i] = kx[i] * e1;
                    qr[i] = qx[i] * e1;
                    kb[i] = kx[i] * e2;
                    rhs[e][i] = br * kr[i] * pm[i];
                }
                st8f<T>(Kr + r * SM::KS + kc0, kr);
                st8f<T>(Qr + r * SM::KS + kc0, qr);
                st8f<T>(Kb + r * SM::KS + kc0, kb);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) st2<T>(RK + krp * SM::RKS + 2 * (kc0 + i), rhs[0][i], rhs[1][i]);
        }
        if (more) load_inputs(nxt, pf, LD_KQ);
        if (val_task) {
            const int s0 = 2 * vrp;
            float vx0[8], vx1[8];
            pf.v[0].get(vx0);
            pf.v[1].get(vx1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                vx0[i] = s0 < nr ? vx0[i] : 0.f;
                vx1[i] = s0 + 1 < nr ? vx1[i] : 0.f;
            }
            const float b0 = Bt[s0], b1 = Bt[s0 + 1];
#pragma unroll
            for (int i = 0; i < 8; ++i) st2<T>(RV + vrp * SM::RVS + 2 * (vc0 + i), b0 * vx0[i], b1 * vx1[i]);
        }
        if (more) load_inputs(nxt, pf, LD_V);
        lds_barrier();

        // ---- P2: decayed K K^T (-> L) and (Q K^T)^T (-> workspace) on MFMA ----------
        // waves 0-5: one off-diagonal tile (R, S) each (f = fp_index(R, S) = wave);
        // waves 6, 7: two diagonal tiles each, which need no decay scaling
        for (int t = 0; t < (wv < 6 ? 1 : 2); ++t) {
            const int R = wv < 6 ? (wv < 1 ? 1 : wv < 3 ? 2 : 3) : 2 * (wv - 6) + t;
            const int S = wv < 6 ? wv - R * (R - 1) / 2 : R;
            f32x4_t accA = zero4(), accB = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c = 32 * ks + 8 * g;
                const F kr = F::ld8(Kr + (16 * R + col) * SM::KS + c);
                const F qr = F::ld8(Qr + (16 * R + col) * SM::KS + c);
                F kb = F::ld8(Kb + (16 * S + col) * SM::KS + c);
                if (S < R) {
                    const float *fp = Fp + fp_index(R, S) * DK + c;
#pragma unroll
                    for (int i = 0; i < 8; ++i) kb.set(i, kb.get(i) * fp[i]);
                }
                accA = mma(kr, kb, accA);   // A[r][s]:  rows r = 16R + 4g + i, column s = 16S + col
                accB = mma(kb, qr, accB);   // Bq[r][s] at rows s = 16S + 4g + i, column r = 16R + col
            }
            float bq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * g + i, s = 16 * S + col;
                Lm[r * SM::LS + s] = s < r ? Bt[r] * accA[i] : 0.f;
                bq[i] = (16 * S + 4 * g + i <= 16 * R + col) ? accB[i] : 0.f;
            }
            st4<T>(ws + WL::BT + ((size_t)(R * 2 + (S >> 1)) * 64 + l) * 8 + (S & 1) * 4, bq);
        }
        if (wv == 2 || wv == 3) {   // the upper sub-blocks (0,1) and (2,3) inside kernel 2's k-steps
            const int R = wv == 2 ? 0 : 2, S = R + 1;
            const float z[4] = {0.f, 0.f, 0.f, 0.f};
            st4<T>(ws + WL::BT + ((size_t)(R * 2 + (S >> 1)) * 64 + l) * 8 + (S & 1) * 4, z);
        }
        lds_barrier();

        // ---- P3: Tm = (I + Diag(beta) A)^-1 in fp32 ------------------------------------
        if (wv == 0) {
            // diagonal blocks by forward substitution: lane = (block R, column j)
            // (four partial sums per row keep the dependent chain short)
            const int R = l >> 4, j = l & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float *Li = Lm + (16 * R + i) * SM::LS + 16 * R;
                float p[4] = {(i == j) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k2 = 0; k2 < i; ++k2) p[k2 & 3] = __builtin_fmaf(-Li[k2], x[k2], p[k2 & 3]);
                x[i] = (p[0] + p[1]) + (p[2] + p[3]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Tm32[(16 * R + i) * SM::LS + 16 * R + j] = x[i];
        } else {
            // waves 1..7: zero the 6 upper sub-blocks of Tm32, then export Kh^T and
            // Qt to the workspace in fragment order (16 contiguous bytes per task)
            if (wv >= 2) {
                const int u = wv - 2;
                const int R = u < 3 ? 0 : u < 5 ? 1 : 2;
                const int S = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
#pragma unroll
                for (int i = 0; i < 4; ++i) Tm32[(16 * R + 4 * g + i) * SM::LS + 16 * S + col] = 0.f;
            }
            constexpr int NT = 8 * DK;   // tasks per tensor: DK/16 * 2 * 64 (Kh) == 4 * DK/32 * 64 (Qt)
            for (int u = tid - 64; u < 2 * NT; u += K1_THREADS - 64) {
                const int v = u < NT ? u : u - NT, ln = v & 63, gq = ln >> 4;
                float x[8];
                if (u < NT) {
                    // Kh^T fragment (dt, kt, lane): channel 16dt + ln%16, tokens
                    // 32kt + 4*(ln/16) + {0..3} (block 2kt) and 32kt + 16 + 4*(ln/16) + {0..3} (block 2kt+1)
                    const int dt = v >> 7, kt = (v >> 6) & 1;
                    const int c = 16 * dt + (ln & 15), t0 = 32 * kt + 4 * gq;
                    const float kh0 = Kh[(2 * kt) * DK + c], kh1 = Kh[(2 * kt + 1) * DK + c];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        x[j] = (float)Kb[(t0 + j) * SM::KS + c] * kh0;
                        x[4 + j] = (float)Kb[(t0 + 16 + j) * SM::KS + c] * kh1;
                    }
                    st8f<T>(ws + WL::KH + (size_t)v * 8, x);
                } else {
                    // Qt fragment (R, ks, lane): row 16R + ln%16, channels 32ks + 4*(ln/16) + {0..3, 16..19}
                    const int R = v / (NKS * 64), ks = (v >> 6) % NKS;
                    const int r = 16 * R + (ln & 15), c0 = 32 * ks + 4 * gq;
                    float a4[4], b4[4];
                    ld4<T>(Qr + r * SM::KS + c0, a4);
                    ld4<T>(Qr + r * SM::KS + c0 + 16, b4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = a4[i] * Pm[R * DK + c0 + i];
                        x[4 + i] = b4[i] * Pm[R * DK + c0 + 16 + i];
                    }
                    st8f<T>(ws + WL::QT + (size_t)v * 8, x);
                }
            }
        }
        lds_barrier();
        // off-diagonal, by distance d = R - S: Tm_RS = -D_R sum_{J=S}^{R-1} L_RJ Tm_JS.
        // Wave S owns block (R, S) of each level; the intermediate sum goes
        // through its own LDS scratch (one wave's LDS accesses complete in
        // order), so only the levels are separated by barriers.
        for (int d = 1; d < 4; ++d) {
            float *sc = Scr + wv * 16 * SM::SC;
            const int R = wv + d, S = wv;
            if (R < 4) {
                f32x4_t y = zero4();
                for (int J = S; J < R; ++J)
                    y = mm16(Lm + (16 * R) * SM::LS + 16 * J, SM::LS, Tm32 + (16 * J) * SM::LS + 16 * S, SM::LS,
                             col, g, y);
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[(4 * g + i) * SM::SC + col] = y[i];
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the scratch writes have completed
                __builtin_amdgcn_wave_barrier();
                const f32x4_t t = mm16(Tm32 + (16 * R) * SM::LS + 16 * R, SM::LS, sc, SM::SC, col, g, zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i) Tm32[(16 * R + 4 * g + i) * SM::LS + 16 * S + col] = -t[i];
            }
            lds_barrier();
        }
        {   // Tm16 <- Tm32
            const int r = tid >> 3, c0 = 8 * (tid & 7);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = Tm32[r * SM::LS + c0 + i];
            st8f<T>(Tm16 + r * SM::TS + c0, x);
        }
        lds_barrier();

        // ---- P5: W^T per 16 key channels, Ut per 16 value columns ------------------
        // Retire the next chunk's prefetch (issued in P1, long since landed) and
        // this chunk's earlier stores here, before P5 issues its own: loads and
        // stores share one counter, so a wait for the prefetch placed after the
        // P5 stores (at the next P0) would also wait for those fresh stores.
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        {
            constexpr int NWU = DK / 16, NUU = DV / 16;
            for (int u = wv; u < NWU + NUU; u += 8) {
                if (u < NWU) {
                    const int at = u;
                    F rk[2];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        rk[ks] = F::ld_pairs(RK + (16 * ks + 4 * g) * SM::RKS + 2 * (16 * at + col), SM::RKS);
#pragma unroll
                    for (int R = 0; R < 4; ++R) {
                        f32x4_t acc = zero4();
#pragma unroll
                        for (int ks = 0; ks <= (R >> 1); ++ks)
                            acc = mma(rk[ks], F::ld8(Tm16 + (16 * R + col) * SM::TS + 32 * ks + 8 * g), acc);
                        const float w4[4] = {acc[0], acc[1], acc[2], acc[3]};
                        st4<T>(ws + WL::W + ((size_t)(R * NKS + (at >> 1)) * 64 + l) * 8 + (at & 1) * 4, w4);
                    }
                } else {
                    const int jt = u - NWU;
                    F rv[2];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        rv[ks] = F::ld_pairs(RV + (16 * ks + 4 * g) * SM::RVS + 2 * (16 * jt + col), SM::RVS);
#pragma unroll
                    for (int R = 0; R < 4; ++R) {
                        f32x4_t acc = zero4();
#pragma unroll
                        for (int ks = 0; ks <= (R >> 1); ++ks)
                            acc = mma(F::ld8(Tm16 + (16 * R + col) * SM::TS + 32 * ks + 8 * g), rv[ks], acc);
                        const float u4[4] = {acc[0], acc[1], acc[2], acc[3]};
                        st4<T>(ws + WL::U + ((size_t)(jt * 64 + l) * 4 + R) * 4, u4);
                    }
                }
            }
        }
        lds_barrier();   // LDS is reused by the next chunk
    }
}

// ---- kernel 2: sequential state pass ------------------------------------------------
// One 7-wave workgroup per (batch, head, 16 value columns):
//   wave 0 (recurrence): S <- Diag(Gam) S + Kh^T (Ut - W S), chunk after chunk;
//   waves 1, 2, 3, 5 (output): O^T = S^T Qt^T + U^T Bq^T from the S and U wave 0
//                        used, chunk n on output wave n mod 4;
//   wave 4 (store):      writes O to o;
//   wave 6 (loader):     stages W, Kh^T, Ut and Gam of the coming chunks in LDS.
// Lane l = 16 g + col of wave 0 holds rows 16 dt + 4 g + i (i = 0..3) of
// value column col of S in fp32: S is kept as DK/16 accumulator tiles.  Two
// tiles side by side are directly an MFMA operand whose 32 k-slots are the
// rows 32 ks + {4g+i, 16+4g+i} -- the B operand of W S (k = key channel) and,
// unchanged, the A operand of S^T Qt^T -- so the state never leaves wave 0's
// registers; U becomes an operand the same way (k = token).  The workspace
// fragments are stored in the matching k order.
// Wave 0 hands the bf16 operands of S and U to the output waves, and they the
// output tiles to the store wave, through small LDS rings guarded by counters: a wave waits
// only when its ring is empty (consumer) or full (producer).  Keeping loads
// and stores in different waves lets every wave keep its loads in flight
// across chunk steps: a wave with both outstanding would drain everything at
// each wait.  Each wave streams its operands through registers one chunk ahead.

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

// Wait until an LDS counter reaches target.  Bounded: a kernel-wide poll
// budget (far above what a correct run uses) guarantees that every wave exits
// even if its partner never signals.
__device__ __forceinline__ void wait_counter(int *ctr, int target, int &budget) {
    while (budget > 0 && __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        --budget;
        __builtin_amdgcn_s_sleep(1);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Publish a counter after this wave's earlier LDS writes have completed.
__device__ __forceinline__ void signal_counter(int *ctr, int value) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0) only
    __hip_atomic_store(ctr, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS counter access for a wave that has direct-to-LDS loads in flight.  The
// compiler makes every LDS access of such a wave wait for all of those loads;
// these two touch only the counter, so they are written out (the read waits
// for its own result inside the same block) and the wave keeps its loads in
// flight.  The caller orders them against its loads with explicit waits.
typedef __attribute__((address_space(3))) int lds_int_t;
__device__ __forceinline__ int lds_counter_read(int *ctr) {
    int v;
    const unsigned off = (unsigned)(uintptr_t)(lds_int_t *)ctr;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(off) : "memory");
    return v;
}
__device__ __forceinline__ void lds_counter_write(int *ctr, int value) {
    const unsigned off = (unsigned)(uintptr_t)(lds_int_t *)ctr;
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(off), "v"(value) : "memory");
}
// Bounded wait on an LDS counter (see wait_counter) through lds_counter_read.
__device__ __forceinline__ void wait_counter_dma(int *ctr, int target, int &budget) {
    while (budget > 0 && lds_counter_read(ctr) < target) {
        --budget;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Wave roles of the state pass.  Waves w and w + 4 of a workgroup run on
// the same SIMD, so the store wave (little work) is wave 4, beside the
// recurrence (wave 0); the output waves are 1 and 2, the loaders 3, 5, 6, 7.
constexpr int kOutWaves = 2;          // output waves; chunk n goes to output wave n % kOutWaves
constexpr int kLoaders = 4;           // loader waves; chunk p goes to loader p % kLoaders
constexpr int kStoreWave = 4;
__device__ __forceinline__ int loader_slot(int wave) {   // loader index, or -1
    return wave == 3 ? 0 : wave >= 5 ? wave - 4 : -1;
}
__device__ __forceinline__ int out_slot(int wave) {   // output wave index, or -1
    return wave == 1 || wave == 2 ? wave - 1 : -1;
}
constexpr int kRing = 4;              // chunk steps buffered between recurrence, output, store
static_assert(kRing % kOutWaves == 0, "each ring slot belongs to one output wave");
constexpr int kOpRing = 3;            // chunks of recurrence operands staged in LDS
constexpr int kPollBudget = 1 << 24;  // LDS polls per wave per launch
constexpr int kScanThreads = 512;     // recurrence, two output waves, four loaders, store

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: vmcnt split over
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

template <typename T, int DK, int DV>
struct ScanLds {
    static constexpr int ES = sizeof(T);
    // one staged chunk of recurrence operands: exact copies of the workspace
    // ranges W, Kh^T, this workgroup's Ut slice and Gam
    static constexpr int W_B = 64 * DK * ES;
    static constexpr int K_B = 64 * DK * ES;
    static constexpr int U_B = 64 * 16 * ES;
    static constexpr int G_B = DK * 4;
    static constexpr int OPB = W_B + K_B + U_B + G_B;
    static constexpr int NI = (W_B + 1023) / 1024 + (K_B + 1023) / 1024 + (U_B + 1023) / 1024 + (G_B + 1023) / 1024;
    static_assert(NI < 64, "one staged chunk must fit the vector memory counter");
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kScanThreads) void kda_state_kernel(KdaArgs a) {
    using WL = Ws<T, DK, DV>;
    using SL = ScanLds<T, DK, DV>;
    using F = Frag<T>;
    using B = BufLd<T>;
    constexpr int NJT = DV / 16;     // workgroups per head: one 16-column value slab each
    constexpr int NKS = DK / 32;     // contraction steps over dk
    constexpr int NDT = DK / 16;     // 16-row state tiles
    constexpr unsigned ES = sizeof(T);
    __shared__ __attribute__((aligned(1024))) char op_ring[kOpRing][SL::OPB];
    // per lane: S operands (NKS fragments) then U operands (2 fragments)
    __shared__ F su_ring[kRing][NKS + 2][64];
    __shared__ f32x4_t o_ring[kRing][4][64];
    // counters, each "chunks done" (n + 1 after chunk n):
    //   kSuProd  S/U operands written (recurrence)
    //   kSuCons  + parity: S/U slot read (output wave of that parity)
    //   kOProd   + parity: O tile written (output wave of that parity)
    //   kOCons   O tile read (store)
    //   kOpProd  + loader: chunks staged by that loader, kOpCons operands read (recurrence)
    constexpr int kSuProd = 0, kSuCons = 1, kOProd = kSuCons + kOutWaves, kOCons = kOProd + kOutWaves,
                  kOpProd = kOCons + 1, kOpCons = kOpProd + kLoaders, kNumCtr = kOpCons + 1;
    __shared__ int ctr[kNumCtr];
    if (threadIdx.x < kNumCtr) ctr[threadIdx.x] = 0;
    __syncthreads();

    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int jt = blk % NJT, bh = blk / NJT;
    const int sq = bh / a.H, h = bh % a.H;   // sequence, head
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, col = l & 15, g = l >> 4;
    // this sequence's chunks [c0, c0 + nchunks) and tokens [tok0, tok0 + ntok)
    const int c0 = seq_chk0(a, sq), nchunks = seq_chk0(a, sq + 1) - c0, last = nchunks - 1;
    const int tok0 = seq_tok0(a, sq), ntok = seq_tok0(a, sq + 1) - tok0;
    int budget = kPollBudget;

    // this (batch, head)'s workspace: chunk n at byte n * BYTES (< 4 GiB, checked on the host)
    const char *wsh = static_cast<const char *>(a.ws) + ((size_t)h * seq_chk0(a, a.B) + c0) * WL::BYTES;
    const __amdgpu_buffer_rsrc_t wsr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(wsh), 0, (int)(unsigned)((size_t)nchunks * WL::BYTES), kBufWord3);
    const unsigned lane8 = (unsigned)l * 8 * ES;   // lane's fragment inside a [64][8] block
    auto cbase = [&](int i) { return (unsigned)i * (unsigned)WL::BYTES; };

    if (loader_slot(wave) >= 0) {
        // ---------------- loaders: recurrence operands -> LDS ----------------
        // Loader q takes chunks p = q, q + kLoaders, ...: it loads the chunk's
        // W, Kh^T, Ut slice and Gam into its registers (16 bytes per lane,
        // 1 KB per instruction), waits until the chunk's ring slot is free,
        // copies the registers into the slot and signals, then loads its next
        // chunk.  With kLoaders waves each holding a chunk in flight, the loads
        // of chunk p are issued about kLoaders + kOpRing - 1 chunk steps before
        // the recurrence reads it, which covers the memory latency.
        const int q = loader_slot(wave);
        u32x4_t r[SL::NI];
        int nload = 0;   // chunks this loader has staged
        auto load = [&](int p) {
            const unsigned c = cbase(p);
            int k = 0;
            auto seg = [&](unsigned src, int bytes) {
#pragma unroll
                for (int i = 0; i < (bytes + 1023) / 1024; ++i, ++k)
                    r[k] = __builtin_amdgcn_raw_buffer_load_b128(wsr, src + (unsigned)(i * 1024 + l * 16), c, 0);
            };
            seg((unsigned)(WL::W * ES), SL::W_B);
            seg((unsigned)(WL::KH * ES), SL::K_B);
            seg((unsigned)((WL::U + (size_t)jt * 64 * 16) * ES), SL::U_B);
            seg((unsigned)WL::GAM_BYTE, SL::G_B);
        };
        auto stage = [&](int p) {
            char *slot = op_ring[p % kOpRing];
            int k = 0;
            auto seg = [&](int off, int bytes) {
#pragma unroll
                for (int i = 0; i < (bytes + 1023) / 1024; ++i, ++k)
                    if (i * 1024 + l * 16 < bytes)
                        *reinterpret_cast<u32x4_t *>(slot + off + i * 1024 + l * 16) = r[k];
            };
            seg(0, SL::W_B);
            seg(SL::W_B, SL::K_B);
            seg(SL::W_B + SL::K_B, SL::U_B);
            seg(SL::W_B + SL::K_B + SL::U_B, SL::G_B);
        };
#pragma unroll 1
        for (int p = q; p < nchunks; p += kLoaders) {
            load(p);
            if (p >= kOpRing) wait_counter(&ctr[kOpCons], p - kOpRing + 1, budget);   // slot's last chunk read
            stage(p);
            signal_counter(&ctr[kOpProd + q], ++nload);
        }
    } else if (wave == 0) {
        // ---------------- recurrence ----------------
        f32x4_t S[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[dt] = zero4();
        if (a.s0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[dt][i] = a.s0[((size_t)bh * DK + 16 * dt + 4 * g + i) * DV + 16 * jt + col];
        }
        // Operands of one chunk in registers, refilled from the LDS ring phase
        // by phase as soon as the current chunk has issued its last use: W after
        // the U products, Kh^T, Ut and Gam after the state update.  Every LDS
        // poll and signal waits for all of this wave's LDS operations, so they
        // come before the refills in each step.
        F Wf[4][NKS], Kf[NDT][2];
        Raw8<T> ut[2];   // Ut rows 16R + 4g + i of column col: element 4R + i
        float2 gam;      // decay of channels 16 dt + 4g + i for dt = col/2, i = 2(col%2) + {0, 1}
        auto read_w = [&](int n) {
            const char *op = op_ring[n % kOpRing];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    Wf[R][ks] = *reinterpret_cast<const F *>(op + (R * NKS + ks) * 64 * 8 * ES + lane8);
        };
        auto read_k = [&](int n) {
            const char *op = op_ring[n % kOpRing];
            ut[0] = *reinterpret_cast<const Raw8<T> *>(op + SL::W_B + SL::K_B + l * 16 * ES);
            ut[1] = *reinterpret_cast<const Raw8<T> *>(op + SL::W_B + SL::K_B + l * 16 * ES + 8 * ES);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    Kf[dt][kt] = *reinterpret_cast<const F *>(op + SL::W_B + (dt * 2 + kt) * 64 * 8 * ES + lane8);
            gam = *reinterpret_cast<const float2 *>(op + SL::W_B + SL::K_B + SL::U_B +
                                                    4 * (g * (DK / 4) + 2 * min(col, DK / 8 - 1)));
        };
        // chunk n is staged once loader n % kLoaders has staged n / kLoaders + 1 chunks
        auto wait_staged = [&](int n) { wait_counter(&ctr[kOpProd + n % kLoaders], n / kLoaders + 1, budget); };
        wait_staged(0);
        read_w(0);
        read_k(0);
#pragma unroll 1
        for (int n = 0; n < nchunks; ++n) {
            // Critical chain of a step: pack S -> U MFMAs -> U = Ut - W S, pack
            // -> state MFMAs.  The decay of S, the ring traffic and the operand
            // refills sit in the shadow of the MFMAs.
            F Sb[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) Sb[ks] = tiles_to_frag<T>(S[2 * ks], S[2 * ks + 1]);
            // U = Ut - W S  (token rows 16R + 4g + i, value column col)
            f32x4_t U[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) U[R] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int R = 0; R < 4; ++R) U[R] = mma(Wf[R][ks], Sb[ks], U[R]);
            // S <- Diag(Gam) S; the decay of (dt, i) sits in lane 2dt + i/2 of the row
            const float2 gm = gam;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[dt][i] *= row_bcast(i & 1 ? gm.y : gm.x, 2 * dt + (i >> 1));
                pin(S[dt]);   // keeps the decay here, under the MFMAs, rather than next to its use
            }
            float x[2][8];
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                ut[R].get(x[R]);
#pragma unroll
                for (int i = 0; i < 8; ++i) pin(x[R][i]);
            }
            // su slot n % kRing is free once chunk n-kRing has been read by the
            // output wave of its parity (kRing is even)
            if (n >= kRing) wait_counter(&ctr[kSuCons + n % kOutWaves], n + 1 - kRing, budget);
            F(&slot)[NKS + 2][64] = su_ring[n % kRing];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) slot[ks][l] = Sb[ks];
#pragma unroll
            for (int R = 0; R < 2; ++R)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    U[2 * R][i] = x[R][i] - U[2 * R][i];
                    U[2 * R + 1][i] = x[R][4 + i] - U[2 * R + 1][i];
                }
            const F Ub[2] = {tiles_to_frag<T>(U[0], U[1]), tiles_to_frag<T>(U[2], U[3])};
            // S <- S + Kh^T U
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) S[dt] = mma(Kf[dt][kt], Ub[kt], S[dt]);
            slot[NKS][l] = Ub[0];
            slot[NKS + 1][l] = Ub[1];
            signal_counter(&ctr[kSuProd], n + 1);
            // chunk n's operands are all in registers: its ring slot may be restaged
            signal_counter(&ctr[kOpCons], n + 1);
            if (n + 1 < nchunks) {
                wait_staged(n + 1);
                read_w(n + 1);
                read_k(n + 1);
            }
        }
        if (a.sT) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.sT[((size_t)bh * DK + 16 * dt + 4 * g + i) * DV + 16 * jt + col] = S[dt][i];
        }
    } else if (out_slot(wave) >= 0) {
        // ---------------- output: O^T = S^T Qt^T + U^T Bq^T ----------------
        // The output waves take chunks in turn.  Each holds the Qt and Bq
        // operands of its next two chunks in two register sets, so their loads
        // go out 2 * kOutWaves chunk steps before use.
        const int par = out_slot(wave);
        F Qa[4][NKS], Ba[6], Qb[4][NKS], Bb[6];
        auto load_qb = [&](int n, F (&Qf)[4][NKS], F (&Bf)[6]) {
            const unsigned c = cbase(n);
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    Qf[R][ks] = B::frag(wsr, lane8, c + (unsigned)(WL::QT + (R * NKS + ks) * 512) * ES);
            // Bq: k-step 0 of every token block, k-step 1 of blocks 2 and 3
#pragma unroll
            for (int R = 0; R < 4; ++R) Bf[R] = B::frag(wsr, lane8, c + (unsigned)(WL::BT + (R * 2) * 512) * ES);
            Bf[4] = B::frag(wsr, lane8, c + (unsigned)(WL::BT + 5 * 512) * ES);
            Bf[5] = B::frag(wsr, lane8, c + (unsigned)(WL::BT + 7 * 512) * ES);
        };
        // one chunk with the operand set (Qf, Bf), which is then reloaded with
        // chunk n + 2 * kOutWaves (clamped: the load count per chunk stays fixed)
        auto chunk = [&](int n, F (&Qf)[4][NKS], F (&Bf)[6]) {
            const bool live = n < nchunks;
            f32x4_t O[4];
            if (live) {
                wait_counter(&ctr[kSuProd], n + 1, budget);
                F(&slot)[NKS + 2][64] = su_ring[n % kRing];
                F Sb[NKS], Ub[2];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) Sb[ks] = slot[ks][l];
                Ub[0] = slot[NKS][l];
                Ub[1] = slot[NKS + 1][l];
#pragma unroll
                for (int R = 0; R < 4; ++R) O[R] = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int R = 0; R < 4; ++R) O[R] = mma(Sb[ks], Qf[R][ks], O[R]);
                // causal inside the chunk: token block R sees token k-steps kt <= R/2
#pragma unroll
                for (int R = 0; R < 4; ++R) O[R] = mma(Ub[0], Bf[R], O[R]);
                O[2] = mma(Ub[1], Bf[4], O[2]);
                O[3] = mma(Ub[1], Bf[5], O[3]);
                signal_counter(&ctr[kSuCons + par], n + 1);   // slot reads are complete (the MFMAs consumed them)
            }
            __builtin_amdgcn_sched_barrier(0);
            load_qb(min(n + 2 * kOutWaves, last), Qf, Bf);
            __builtin_amdgcn_sched_barrier(0);
            if (live) {
                if (n >= kRing) wait_counter(&ctr[kOCons], n + 1 - kRing, budget);
#pragma unroll
                for (int R = 0; R < 4; ++R) o_ring[n % kRing][R][l] = O[R];
                signal_counter(&ctr[kOProd + par], n + 1);
            }
        };
        load_qb(min(par, last), Qa, Ba);
        __builtin_amdgcn_sched_barrier(0);
        load_qb(min(par + kOutWaves, last), Qb, Bb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
        for (int n = par; n < nchunks; n += 2 * kOutWaves) {
            chunk(n, Qa, Ba);
            chunk(n + kOutWaves, Qb, Bb);
        }
    } else if (wave == kStoreWave) {
        // ---------------- store ----------------
        // o of this (batch, head, 16 value columns) as a raw buffer: token t at
        // byte t*H*DV*es.  Rows past the end of the stream fall outside the range
        // and the hardware drops their stores.  The output tile is transposed
        // (lane: 4 consecutive value columns of one token).
        const unsigned orow = (unsigned)a.H * DV * ES;
        char *obase = static_cast<char *>(a.o) + (((size_t)tok0 * a.H + h) * DV + 16 * jt) * ES;
        const unsigned onum = (unsigned)ntok * orow - (unsigned)(h * DV + 16 * jt) * ES;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(obase, 0, (int)onum, kBufWord3);
        const unsigned ovoff = (unsigned)col * orow + (unsigned)(4 * g) * ES;
#pragma unroll 1
        for (int n = 0; n < nchunks; ++n) {
            wait_counter(&ctr[kOProd + n % kOutWaves], n + 1, budget);
            f32x4_t O[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) O[R] = o_ring[n % kRing][R][l];
            signal_counter(&ctr[kOCons], n + 1);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const unsigned soff = ((unsigned)n * C + 16u * R) * orow;
                if (sizeof(T) == 2) {
                    u32x2_t v;
                    v[0] = pack_bf16x2(O[R][0], O[R][1]);
                    v[1] = pack_bf16x2(O[R][2], O[R][3]);
                    __builtin_amdgcn_raw_buffer_store_b64(v, orsrc, ovoff, soff, 0);
                } else {
                    u32x4_t v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(O[R][i]);
                    __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, ovoff, soff, 0);
                }
            }
        }
    }
}

template <typename T, int DK, int DV>
hipError_t launch_chunks_typed(const KdaArgs &a, hipStream_t stream) {
    using SM = K1Smem<T, DK, DV>;
    static bool attr_set = false;   // per process; setting it twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kda_intra_kernel<T, DK, DV>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)SM::BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int items = a.H * seq_chk0(a, a.B);
    const int grid = items < num_cus() ? items : num_cus();
    hipLaunchKernelGGL((kda_intra_kernel<T, DK, DV>), dim3(grid), dim3(K1_THREADS), SM::BYTES, stream, a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_scan_typed(const KdaArgs &a, hipStream_t stream) {
    const int n2 = a.B * a.H * (DV / 16);
    hipLaunchKernelGGL((kda_state_kernel<T, DK, DV>), dim3(n2), dim3(kScanThreads), 0, stream, a);
    return hipGetLastError();
}

#define KDA_DISPATCH(FN)                                                                           \
    if (a.B == 0 || seq_chk0(a, a.B) == 0) return hipSuccess;                                      \
    if (bf16) {                                                                                    \
        if (a.dk == 64 && a.dv == 64) return FN<bf16_t, 64, 64>(a, stream);                        \
        if (a.dk == 64 && a.dv == 128) return FN<bf16_t, 64, 128>(a, stream);                      \
        if (a.dk == 128 && a.dv == 64) return FN<bf16_t, 128, 64>(a, stream);                      \
        if (a.dk == 128 && a.dv == 128) return FN<bf16_t, 128, 128>(a, stream);                    \
    } else {                                                                                       \
        if (a.dk == 64 && a.dv == 64) return FN<float, 64, 64>(a, stream);                         \
    }                                                                                              \
    return hipErrorInvalidValue;

}  // namespace

int num_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}


size_t kda_chunk_ws_bytes(int dk, int dv, bool bf16) {
#define WS_CASE(DK_, DV_)                                                                          \
    if (dk == DK_ && dv == DV_) return bf16 ? Ws<bf16_t, DK_, DV_>::BYTES : Ws<float, DK_, DV_>::BYTES;
    WS_CASE(64, 64)
    WS_CASE(64, 128)
    WS_CASE(128, 64)
    WS_CASE(128, 128)
#undef WS_CASE
    return 0;
}

hipError_t launch_kda_chunks(const KdaArgs &a, bool bf16, hipStream_t stream) {
    KDA_DISPATCH(launch_chunks_typed)
}

hipError_t launch_kda_scan(const KdaArgs &a, bool bf16, hipStream_t stream) {
    KDA_DISPATCH(launch_scan_typed)
}

}  // namespace kdaconv
