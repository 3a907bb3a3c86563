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
#include "kda_ws.h"

namespace kdaconv {
namespace {

constexpr int C = kChunk;          // 64 tokens per chunk
constexpr int K1_THREADS = 512;    // 8 waves


// ---- kernel 1 shared-memory plan --------------------------------------------------
template <typename T, int DK, int DV>
struct K1Smem {
    static constexpr int NPART = K1_THREADS / DK;     // threads per channel in the table loop
    static constexpr int KP = 16 / (int)sizeof(T);
    static constexpr int KS = DK + KP;                // row stride of Kr, Qr, Kb
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
    // RHS_K = Diag(beta) 2^G K and RHS_V = Diag(beta) V as row pairs (P1-P5): in LDS
    // when everything fits, else (fp32 at dk = 128) in the chunk's own record, in
    // the W and Ut slots that P5 overwrites last (row-pair strides 2 dk and 2 dv)
    static constexpr size_t TAB_B = (size_t)(14 * DK + 64) * 4;
    static constexpr size_t RKV_LDS_B = round_up((size_t)32 * 2 * (DK + 8 / sizeof(T)) * sizeof(T), 16) +
                                        round_up((size_t)32 * 2 * (DV + 8 / sizeof(T)) * sizeof(T), 16);
    static constexpr bool RKV_LDS = round_up(Q + round_up(SZ_K, 16) + RKV_LDS_B + TAB_B, 16) <= 160 * 1024;
    static constexpr int RKS = RKV_LDS ? 2 * (DK + 8 / (int)sizeof(T)) : 2 * DK;   // row-pair stride of RHS_K
    static constexpr int RVS = RKV_LDS ? 2 * (DV + 8 / (int)sizeof(T)) : 2 * DV;   // row-pair stride of RHS_V
    static constexpr size_t RK = Q + round_up(SZ_K, 16);
    static constexpr size_t RV = RK + (RKV_LDS ? round_up((size_t)32 * RKS * sizeof(T), 16) : 0);
    static constexpr size_t TB = RV + (RKV_LDS ? round_up((size_t)32 * RVS * sizeof(T), 16) : 0);
    // tables (fp32): Pm[4][DK], Kh[4][DK], Fp[6][DK], beta[64]
    static constexpr size_t TB_PM = TB;
    static constexpr size_t TB_KH = TB_PM + 4 * DK * 4;
    static constexpr size_t TB_FP = TB_KH + 4 * DK * 4;
    static constexpr size_t TB_BETA = TB_FP + 6 * DK * 4;
    static constexpr size_t BYTES = round_up(TB_BETA + 64 * 4, 16);
    // the fused variant (conv in the loader): one head's taps for q, k and v, tap-major
    // [31][DK | DK | DV] in the stream dtype, after everything else, when they fit
    static constexpr size_t CW = BYTES;
    static constexpr size_t CW_BYTES = (size_t)31 * (2 * DK + DV) * sizeof(T);
    static constexpr bool CW_LDS = round_up(CW + CW_BYTES, 16) <= 160 * 1024;
    static constexpr size_t BYTES_CONV = CW_LDS ? round_up(CW + CW_BYTES, 16) : BYTES;
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

// ---- the conv inside the loader (launch_kda_chunks_conv) ----------------------
// The modality-aware depthwise conv of the Chimera core method (genai-atlas "How it
// works"): a text token sums 4 causal taps over the text tokens up to it, a visual
// token the 3x3x3 neighbourhood of its (t, h, w) cell, with zeros outside the grid
// (taps at t-1..t+1, or t-2..t with time-causal padding).  A token's taps are
// walked as 27 slots: visual slot j is tap j = a*9 + b*3 + e; text slot j < 4 is
// tap 27 + j (token tr - 3 + j), and the other slots are empty.
struct ConvPlace {
    int tr;           // stream-relative token
    int ft, fy, fx;   // its grid cell (visual tokens)
    bool text;
};
__device__ __forceinline__ ConvPlace conv_place(const KdaArgs &a, int tr) {
    ConvPlace P;
    P.tr = tr;
    P.text = tr < a.n_text;
    const int p = P.text ? 0 : tr - a.n_text, hw = a.gh * a.gw;
    P.ft = hw ? p / hw : 0;
    const int rem = p - P.ft * hw;
    P.fy = a.gw ? rem / a.gw : 0;
    P.fx = rem - P.fy * a.gw;
    return P;
}
// Slot j of a token: the token it reads (the token itself for an empty slot, whose
// term is dropped, so every load is in bounds and none waits on a branch), the tap
// (its weight row) and whether the term counts.
__device__ __forceinline__ int conv_slot(const KdaArgs &a, const ConvPlace &P, int j, int &tap, bool &ok) {
    if (P.text) {
        const int t = P.tr - 3 + j;
        ok = j < 4 && t >= 0;
        tap = 27 + (j < 4 ? j : 0);
        return ok ? t : P.tr;
    }
    const int ta = j / 9, tb = (j / 3) % 3, te = j % 3;
    const int tt = P.ft + ta - a.pt, yy = P.fy + tb - 1, xx = P.fx + te - 1;
    ok = tt >= 0 && tt < a.gt && yy >= 0 && yy < a.gh && xx >= 0 && xx < a.gw;
    tap = j;
    return ok ? a.n_text + (tt * a.gh + yy) * a.gw + xx : P.tr;
}
// One conv output row of 8 channels: its stream's tokens (of one sequence) through a
// buffer resource, C channels per token, channel c0 of the row at element xo of a
// token, and of tap 0 at element wo of the tap-major taps.
struct ConvRow {
    __amdgpu_buffer_rsrc_t x;
    int C, xo, wo;   // wo: taps in global memory (element offset of tap 0, channel c0; C per tap)
    int lo, D;       // or in LDS: element offset of tap 0, channel c0, and D per tap
    ConvPlace P;
};
// NO output rows at once, TPR slots per round: each round issues all its loads (the
// rows' neighbours and taps, one 32-bit offset each) before the first multiply-add.
// fp32 sums in slot order, rounded to T.
template <typename T, int NO, int TPR, bool WLDS>
__device__ __forceinline__ void conv_rows(const KdaArgs &a, __amdgpu_buffer_rsrc_t wr, const T *wl,
                                          const ConvRow (&o)[NO], Raw8<T> (&out)[NO]) {
    static_assert(27 % TPR == 0, "whole rounds of slots");
    constexpr unsigned ES = sizeof(T);
    float acc[NO][8];
#pragma unroll
    for (int n = 0; n < NO; ++n)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[n][i] = 0.f;
#pragma unroll 1
    for (int j0 = 0; j0 < 27; j0 += TPR) {
        Raw8<T> xv[NO][TPR], wv[NO][TPR];
        bool okv[NO][TPR];
        int tapv[NO][TPR];
#pragma unroll
        for (int u = 0; u < TPR; ++u)
#pragma unroll
            for (int n = 0; n < NO; ++n) {
                const int tok = conv_slot(a, o[n].P, j0 + u, tapv[n][u], okv[n][u]);
                xv[n][u].load_buf(o[n].x, (unsigned)(tok * o[n].C + o[n].xo) * ES);
                if constexpr (!WLDS) wv[n][u].load_buf(wr, (unsigned)(tapv[n][u] * o[n].C + o[n].wo) * ES);
            }
#pragma unroll
        for (int u = 0; u < TPR; ++u)
#pragma unroll
            for (int n = 0; n < NO; ++n) {
                // taps in LDS are read where they are used: a round holds only its inputs
                if constexpr (WLDS) wv[n][u].load(wl + tapv[n][u] * o[n].D + o[n].lo);
                float xf[8], wf[8];
                xv[n][u].get(xf);
                wv[n][u].get(wf);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[n][i] = fmaf(okv[n][u] ? wf[i] : 0.f, xf[i], acc[n][i]);
            }
    }
#pragma unroll
    for (int n = 0; n < NO; ++n) out[n].set(acc[n]);
}

// Two consecutive visual rows, tokens P0.tr and P0.tr + 1 of one sequence (the pair of rows
// a thread consumes in P1), of NT tensors, with the taps in LDS (RW elements per tap).  The
// neighbour (t + a - pt, h + b - 1, w + e - 1) of token tr is token tr + off + e - 1 with
// off = (a - pt) h w + (b - 1) w wherever it lies in the grid, so for each (a, b) the three
// e taps of both rows read the 4 tokens P0.tr + off - 1 .. P0.tr + off + 2: 4 NT loads a
// round, 9 rounds.  Tokens outside the stream are clamped into it (only empty taps read
// them).  A second row past the chunk's end repeats the first (P1 = P0): it is formed from
// the wrong tokens and dropped where it is used.
template <typename T, int NT>
__device__ __forceinline__ void conv_pair_visual(const KdaArgs &a, const T *wl, int RW, const ConvPlace &P0,
                                                 const ConvPlace &P1, const ConvRow (&o)[NT],
                                                 Raw8<T> (&out)[NT][2]) {
    constexpr unsigned ES = sizeof(T);
    float acc[NT][2][8];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[n][0][i] = acc[n][1][i] = 0.f;
    const int hw = a.gh * a.gw, last = a.T - 1;
#pragma unroll 1
    for (int ab = 0; ab < 9; ++ab) {
        const int ta = ab / 3, tb = ab - 3 * ta;
        const int base = P0.tr + (ta - a.pt) * hw + (tb - 1) * a.gw - 1;
        Raw8<T> xv[NT][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int tok = min(max(base + q, 0), last);
#pragma unroll
            for (int n = 0; n < NT; ++n) xv[n][q].load_buf(o[n].x, (unsigned)(tok * o[n].C + o[n].xo) * ES);
        }
        const int tt0 = P0.ft + ta - a.pt, yy0 = P0.fy + tb - 1, tt1 = P1.ft + ta - a.pt, yy1 = P1.fy + tb - 1;
        const bool in0 = tt0 >= 0 && tt0 < a.gt && yy0 >= 0 && yy0 < a.gh;
        const bool in1 = tt1 >= 0 && tt1 < a.gt && yy1 >= 0 && yy1 < a.gh;
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            const bool ok0 = in0 && P0.fx + e - 1 >= 0 && P0.fx + e - 1 < a.gw;
            const bool ok1 = in1 && P1.fx + e - 1 >= 0 && P1.fx + e - 1 < a.gw;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                Raw8<T> w;
                w.load(wl + (ab * 3 + e) * RW + o[n].lo);
                float wf[8], x0[8], x1[8];
                w.get(wf);
                xv[n][e].get(x0);
                xv[n][e + 1].get(x1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc[n][0][i] = fmaf(ok0 ? wf[i] : 0.f, x0[i], acc[n][0][i]);
                    acc[n][1][i] = fmaf(ok1 ? wf[i] : 0.f, x1[i], acc[n][1][i]);
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        out[n][0].set(acc[n][0]);
        out[n][1].set(acc[n][1]);
    }
}

template <typename T, int DK, int DV, bool CONV = false>
__global__ __launch_bounds__(K1_THREADS) void kda_intra_kernel(KdaArgs a) {
    using SM = K1Smem<T, DK, DV>;
    using WL = Ws<T, DK, DV>;
    using F = Frag<T>;
    static_assert(SM::BYTES <= 160 * 1024 && SM::BYTES_CONV <= 160 * 1024, "LDS plan exceeds 160 KB");
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
        int sq, tr0;   // sequence and stream-relative first token (uniform batch; the conv loader)
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
            if constexpr (CONV) {
                L.sq = sq;
                L.tr0 = n * C;
            }
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
    T *const RK_lds = reinterpret_cast<T *>(smem + SM::RK);
    T *const RV_lds = reinterpret_cast<T *>(smem + SM::RV);
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
        if constexpr (!CONV) {   // (with the conv, q', k', v' come from conv_inputs)
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
        }
    };

    // The conv inside the loader: q', k', v' of chunk L's rows (the rows this thread
    // consumes in P1, rows past the end repeating the last row) formed from the conv
    // inputs, at the top of the chunk's iteration, where little else is live.
    // (with SM::CW_LDS the head's taps sit in LDS, copied there when the head changes)
    T *const cw_lds = reinterpret_cast<T *>(smem + SM::CW);
    int cw_head = -1;
    auto conv_inputs = [&](const Loc &L, Prefetch<T> &pf) {
        const int h = L.h, nr = L.nr;
        const int CK = a.H * DK, CV = a.H * DV;
        const size_t tk = (size_t)a.T * CK, tv = (size_t)a.T * CV;   // one sequence of a stream, elements
        // the item's sequence of each stream (the same for every lane) and the taps
        auto rsrc = [](const void *p, size_t bytes) {
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)(unsigned)bytes, kBufWord3);
        };
        const __amdgpu_buffer_rsrc_t wr = rsrc(a.cw, (size_t)kConvTaps * (2 * CK + CV) * sizeof(T));
        if constexpr (SM::CW_LDS) {
            if (h != cw_head) {   // uniform: every lane holds the same item
                // LDS row j of stream s: [s = 0: q | 1: k | 2: v] at (j * (2 DK + DV) + s * DK)
                constexpr int RW = 2 * DK + DV, PIECES = kConvTaps * RW / 8;
                const T *g = static_cast<const T *>(a.cw);
                for (int pc = tid; pc < PIECES; pc += K1_THREADS) {
                    const int j = pc / (RW / 8), e = 8 * (pc - j * (RW / 8));
                    const int st = e < DK ? 0 : (e < 2 * DK ? 1 : 2);
                    const int c = e - st * DK, Cs = st < 2 ? CK : CV, D = st < 2 ? DK : DV;
                    Raw8<T> w;
                    w.load(g + a.cw_off[st] + (size_t)j * Cs + h * D + c);
                    *reinterpret_cast<Raw8<T> *>(cw_lds + j * RW + e) = w;
                }
                __syncthreads();
                cw_head = h;
            }
        }
        // every thread forms two rows of k, q and v; a thread past the value rows
        // (dv < dk) forms rows of its clamped place too and drops them
        const __amdgpu_buffer_rsrc_t rk = rsrc(k_in + (size_t)L.sq * tk, tk * sizeof(T));
        const __amdgpu_buffer_rsrc_t rq = rsrc(q_in + (size_t)L.sq * tk, tk * sizeof(T));
        const __amdgpu_buffer_rsrc_t rv = rsrc(v_in + (size_t)L.sq * tv, tv * sizeof(T));
        const int xk = h * DK + kc0, xv = h * DV + vc0, RW = 2 * DK + DV;
        const ConvPlace P0 = conv_place(a, L.tr0 + min(2 * krp, nr - 1));
        const ConvPlace P1 = conv_place(a, L.tr0 + min(2 * krp + 1, nr - 1));
        const ConvPlace V0 = conv_place(a, L.tr0 + min(2 * vrp, nr - 1));
        const ConvPlace V1 = conv_place(a, L.tr0 + min(2 * vrp + 1, nr - 1));
        const ConvRow rk2[2] = {{rk, CK, xk, a.cw_off[1] + xk, DK + kc0, RW, P0},
                                {rk, CK, xk, a.cw_off[1] + xk, DK + kc0, RW, P1}};
        const ConvRow rq2[2] = {{rq, CK, xk, a.cw_off[0] + xk, kc0, RW, P0}, {rq, CK, xk, a.cw_off[0] + xk, kc0, RW, P1}};
        const ConvRow rv2[2] = {{rv, CV, xv, a.cw_off[2] + xv, 2 * DK + vc0, RW, V0},
                                {rv, CV, xv, a.cw_off[2] + xv, 2 * DK + vc0, RW, V1}};
        // as many loads per round as the registers left at the top of the iteration hold
        // without spilling; a visual pair of rows shares its neighbours (conv_pair_visual),
        // and at dk = dv the k, q and v rows are the same two tokens
        Raw8<T> res_v[2];
        if constexpr (SM::CW_LDS && DK == DV) {
            if (!P0.text) {
                const ConvRow r3[3] = {rk2[0], rq2[0], rv2[0]};
                Raw8<T> res[3][2];
                conv_pair_visual<T, 3>(a, cw_lds, RW, P0, P1, r3, res);
                pf.k[0] = res[0][0];
                pf.k[1] = res[0][1];
                pf.q[0] = res[1][0];
                pf.q[1] = res[1][1];
                res_v[0] = res[2][0];
                res_v[1] = res[2][1];
            } else {   // text rows (the first chunks of a stream): slot by slot
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rk2, pf.k);
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rq2, pf.q);
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rv2, res_v);
            }
        } else if constexpr (SM::CW_LDS) {
            if (!P0.text) {
                const ConvRow rkq[2] = {rk2[0], rq2[0]};
                Raw8<T> res[2][2];
                conv_pair_visual<T, 2>(a, cw_lds, RW, P0, P1, rkq, res);
                pf.k[0] = res[0][0];
                pf.k[1] = res[0][1];
                pf.q[0] = res[1][0];
                pf.q[1] = res[1][1];
            } else {
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rk2, pf.k);
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rq2, pf.q);
            }
            if (!V0.text) {
                const ConvRow rv1[1] = {rv2[0]};
                Raw8<T> res[1][2];
                conv_pair_visual<T, 1>(a, cw_lds, RW, V0, V1, rv1, res);
                res_v[0] = res[0][0];
                res_v[1] = res[0][1];
            } else {
                conv_rows<T, 2, 3, true>(a, wr, cw_lds, rv2, res_v);
            }
        } else if constexpr (sizeof(T) == 2) {
            const ConvRow rkq[4] = {rk2[0], rk2[1], rq2[0], rq2[1]};
            Raw8<T> res[4];
            conv_rows<T, 4, 1, false>(a, wr, cw_lds, rkq, res);
            pf.k[0] = res[0];
            pf.k[1] = res[1];
            pf.q[0] = res[2];
            pf.q[1] = res[3];
            conv_rows<T, 2, 1, false>(a, wr, cw_lds, rv2, res_v);
        } else {
            conv_rows<T, 2, 1, false>(a, wr, cw_lds, rk2, pf.k);
            conv_rows<T, 2, 1, false>(a, wr, cw_lds, rq2, pf.q);
            conv_rows<T, 2, 1, false>(a, wr, cw_lds, rv2, res_v);
        }
        if (val_task) {
            pf.v[0] = res_v[0];
            pf.v[1] = res_v[1];
        }
    };

    Prefetch<T> pf;
    int item = blockIdx.x;
    Loc nxt{0, 0, 0, 0, 0, 0};   // the chunk whose inputs are in the prefetch registers
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
        if constexpr (CONV) conv_inputs(cur, pf);
        const bool more = item + (int)gridDim.x < n_items;
        if (more) nxt = locate(item + gridDim.x);
        char *wsb = static_cast<char *>(a.ws) + ((size_t)cur.h * total + cur.gc) * WL::BYTES;
        T *ws = reinterpret_cast<T *>(wsb);
        T *const RK = SM::RKV_LDS ? RK_lds : ws + WL::W;
        T *const RV = SM::RKV_LDS ? RV_lds : ws + WL::U;
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
            static_assert(NWU + NUU <= 16, "at most two P5 units per wave");
            // unit u < NWU: W^T rows of key channels 16 u ..; else Ut columns 16 (u - NWU) ..
            auto load_unit = [&](int u, F (&op)[2]) {
                const bool wu = u < NWU;
                const int c16 = 16 * (wu ? u : u - NWU) + col;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    op[ks] = wu ? F::ld_pairs(RK + (16 * ks + 4 * g) * SM::RKS + 2 * c16, SM::RKS)
                                : F::ld_pairs(RV + (16 * ks + 4 * g) * SM::RVS + 2 * c16, SM::RVS);
            };
            auto compute_unit = [&](int u, const F (&op)[2]) {
                if (u < NWU) {
                    const int at = u;
#pragma unroll
                    for (int R = 0; R < 4; ++R) {
                        f32x4_t acc = zero4();
#pragma unroll
                        for (int ks = 0; ks <= (R >> 1); ++ks)
                            acc = mma(op[ks], F::ld8(Tm16 + (16 * R + col) * SM::TS + 32 * ks + 8 * g), acc);
                        const float w4[4] = {acc[0], acc[1], acc[2], acc[3]};
                        st4<T>(ws + WL::W + ((size_t)(R * NKS + (at >> 1)) * 64 + l) * 8 + (at & 1) * 4, w4);
                    }
                } else {
                    const int jt = u - NWU;
#pragma unroll
                    for (int R = 0; R < 4; ++R) {
                        f32x4_t acc = zero4();
#pragma unroll
                        for (int ks = 0; ks <= (R >> 1); ++ks)
                            acc = mma(F::ld8(Tm16 + (16 * R + col) * SM::TS + 32 * ks + 8 * g), op[ks], acc);
                        const float u4[4] = {acc[0], acc[1], acc[2], acc[3]};
                        st4<T>(ws + WL::U + ((size_t)(jt * 64 + l) * 4 + R) * 4, u4);
                    }
                }
            };
            if constexpr (SM::RKV_LDS) {
                for (int u = wv; u < NWU + NUU; u += 8) {
                    F op[2];
                    load_unit(u, op);
                    compute_unit(u, op);
                }
            } else {
                // RHS_K and RHS_V sit in the W and Ut slots the results overwrite.  Wave
                // w owns W unit w and Ut unit w + 8 (dk = 128).  Every wave's P1 stores
                // are visible after the first barrier; every wave holds its RHS_K operands
                // before the second lets W be stored; no Ut is stored before the third,
                // so the RHS_V reads between the two can still find their values.
                static_assert(NWU == 8, "the record slots stand in for LDS only at dk = 128");
                __syncthreads();
                F op[2];
                load_unit(wv, op);
                __syncthreads();
                compute_unit(wv, op);
                const bool has_u = wv + 8 < NWU + NUU;
                if (has_u) load_unit(wv + 8, op);
                __syncthreads();
                if (has_u) compute_unit(wv + 8, op);
            }
        }
        lds_barrier();   // LDS is reused by the next chunk
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
hipError_t launch_chunks_conv_typed(const KdaArgs &a, hipStream_t stream) {
    using SM = K1Smem<T, DK, DV>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kda_intra_kernel<T, DK, DV, true>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)SM::BYTES_CONV);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int items = a.H * seq_chk0(a, a.B);
    const int grid = items < num_cus() ? items : num_cus();
    hipLaunchKernelGGL((kda_intra_kernel<T, DK, DV, true>), dim3(grid), dim3(K1_THREADS), SM::BYTES_CONV, stream,
                       a);
    return hipGetLastError();
}

// Taps to tap-major: one thread per (stream, tap, channel).
struct TapArgs {
    const void *wt[3], *wv[3];
    void *cw;
    int C[3], off[3];
};
template <typename T>
__global__ __launch_bounds__(256) void conv_taps_kernel(TapArgs a) {
    int i = blockIdx.x * 256 + threadIdx.x;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int n = kConvTaps * a.C[s];
        if (i >= 0 && i < n) {
            const int tap = i / a.C[s], c = i - tap * a.C[s];
            const T *src = tap < 27 ? static_cast<const T *>(a.wv[s]) + (size_t)c * 27 + tap
                                    : static_cast<const T *>(a.wt[s]) + (size_t)c * 4 + (tap - 27);
            static_cast<T *>(a.cw)[a.off[s] + i] = *src;
        }
        i -= n;
    }
}



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

hipError_t launch_kda_chunks_conv(const KdaArgs &a, bool bf16, hipStream_t stream) {
    if (a.varlen) return hipErrorInvalidValue;
    KDA_DISPATCH(launch_chunks_conv_typed)
}

hipError_t launch_conv_taps_tapmajor(const void *const wt[3], const void *const wv[3], const int Cs[3],
                                     const int off[3], void *cw, bool bf16, hipStream_t stream) {
    TapArgs a;
    int64_t total = 0;
    for (int s = 0; s < 3; ++s) {
        a.wt[s] = wt[s];
        a.wv[s] = wv[s];
        a.C[s] = Cs[s];
        a.off[s] = off[s];
        total += (int64_t)kConvTaps * Cs[s];
    }
    a.cw = cw;
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL(conv_taps_kernel<bf16_t>, dim3(blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(conv_taps_kernel<float>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kdaconv
