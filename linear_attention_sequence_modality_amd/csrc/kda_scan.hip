// Inter-chunk state pass of the chunked KDA forward for gfx950, cut into
// segments that run in parallel.
//
// Per (sequence, head), chunk n of the workspace (formed by the chunk
// transform) maps the state S_n (dk x dv, fp32) to
//   U_n = Ut_n - W_n S_n,   O_n = Qt_n S_n + Bq_n U_n,
//   S_{n+1} = Diag(Gam_n) S_n + Kh_n^T U_n
// which is the gated delta rule S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
// + beta_t k_t v_t^T, o_t = S_t^T q_t (Chimera, method step (5)) regrouped by
// chunks of 64 tokens.  The chunk map is affine in S, so a run of chunks maps
// its start state S to Phi S + L, with Phi (dk x dk) the run's maps applied to
// the identity without the Ut terms, and L (dk x dv) the run started from zero.
//
// Each sequence's chunks are cut into segments of consecutive chunks, and the
// ordered pass becomes three launches:
//   kda_segsum_kernel  every segment but a sequence's last, all in parallel:
//                      one workgroup forms both L and Phi (the "summaries");
//   kda_chain_kernel   per (sequence, head, 16 state columns), in segment
//                      order: S_start(p + 1) = Phi_p S_start(p) + L_p, in fp32;
//   kda_segout_kernel  every segment in parallel, one workgroup per (segment,
//                      head) over all dv columns: replays the segment's chunks
//                      from S_start(p) and writes o, and the final state after
//                      a sequence's last segment.
// The chain is the only serial part and it has one step per segment instead
// of one per chunk; every chunk record is read by one workgroup per pass, not
// once per 16 state columns.
//
// Workgroup layout of the two chunk-walking kernels: compute wave jt owns the
// 16 state columns 16 jt + col.  Lane l = 16 g + col holds rows 16 dt + 4 g + i
// (i = 0..3) of its column as DK/16 fp32 accumulator tiles; two tiles side by
// side are directly a bf16 (or fp32) MFMA operand whose 32 k-slots are the
// rows 32 ks + {4g+i, 16+4g+i}, the order in which the workspace stores W,
// Qt, Kh^T and Bq.  A chunk's shared operands (W, Qt, Kh^T, Bq) are copied into
// an LDS slot with direct-to-LDS buffer loads by a loader wave, one chunk
// ahead into the other slot (the compiler makes every LDS read of a wave wait
// for that wave's own direct-to-LDS loads, so no compute wave issues any);
// a compute wave's own Ut columns and the chunk decay go straight into its
// registers.  One workgroup barrier per chunk (LDS only: vector memory stays
// in flight) publishes the slot.  In the replay a store wave writes o from an
// LDS staging buffer in whole token rows, so the compute waves never have
// stores in flight.
#include "kda_ws.h"

namespace kdaconv {
namespace {

constexpr int kLdsMax = 160 * 1024;   // LDS per workgroup on gfx950
// Launch bounds of the widest instantiations (a bound that depends on the
// template arguments keeps the host pass from emitting the kernel's stub).
constexpr int kSegsumMaxThreads = 64 * (256 / 32 + 1);
constexpr int kSegoutMaxThreads = 64 * (128 / 16 + 2);

// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt at their maxima).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// ---- segment records --------------------------------------------------------
// One per (head, segment), fp32: L and S_start (DK x DV) in state-fragment
// order, Phi (DK x DK) row-major.  State-fragment order holds element (row
// 16 dt + 4 g + i, column 16 jt + col) at ((jt * DK/16 + dt) * 64 + 16 g + col) * 4 + i:
// the four values a lane of the wave owning columns 16 jt .. of a state tile
// holds are 16 contiguous bytes.
template <int DK, int DV>
struct SegRec {
    float *L, *Phi, *S0;
    __device__ SegRec(const KdaArgs &a, int h, int g) {
        const int total = seq_seg0(a, a.B);
        char *r = static_cast<char *>(a.ws) + a.seg_base + ((size_t)h * total + g) * seg_record_bytes(DK, DV);
        L = reinterpret_cast<float *>(r);
        Phi = L + DK * DV;
        S0 = Phi + DK * DK;
    }
};

// Offset (in floats) of lane l's four values of tile (jt, dt) in state-fragment order.
template <int DK>
__device__ __forceinline__ int frag_off(int jt, int dt, int l) { return ((jt * (DK / 16) + dt) * 64 + l) * 4; }

// One (sequence, head)'s chunk records as a raw buffer (chunk n at byte n * BYTES;
// the host checks that a sequence's records stay below 4 GiB).
template <typename T, int DK, int DV>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_records(const KdaArgs &a, int sq, int h) {
    using WL = Ws<T, DK, DV>;
    const int c0 = seq_chk0(a, sq), nch = seq_chk0(a, sq + 1) - c0;
    const char *wsh = static_cast<const char *>(a.ws) + ((size_t)h * seq_chk0(a, a.B) + c0) * WL::BYTES;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(wsh), 0, (int)(unsigned)((size_t)nch * WL::BYTES),
                                             kBufWord3);
}

// Register operands of one chunk for compute wave jt: its Ut columns (rows
// 16R + 4g + i of column col at element 4R + i) and the chunk decay of the
// channels 16 dt + 4g + i for dt = col/2, i = 2(col%2) + {0, 1}.
template <typename T, int DK, int DV>
struct ChunkRegs {
    Raw8<T> ut[2];
    float2 gam;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, unsigned cbase, int jt, int l, bool want_ut) {
        using WL = Ws<T, DK, DV>;
        constexpr unsigned ES = sizeof(T);
        const int col = l & 15, g = l >> 4;
        if (want_ut) {
            const unsigned uo = (unsigned)((WL::U + (size_t)jt * 1024 + (size_t)l * 16) * ES);
            BufLd<T>::raw8(ut[0], r, uo, cbase);
            BufLd<T>::raw8(ut[1], r, uo + 8 * ES, cbase);
        }
        const unsigned go = (unsigned)WL::GAM_BYTE + 4u * (unsigned)(g * (DK / 4) + 2 * min(col, DK / 8 - 1));
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, go, cbase, 0);
        gam = make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
    }
};

// S <- Diag(Gam) S: the decay of row 16 dt + 4g + i sits in lane 2 dt + i/2 of the row of 16.
template <int NDT>
__device__ __forceinline__ void decay_rows(f32x4_t (&S)[NDT], float2 gam) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[dt][i] *= row_bcast(i & 1 ? gam.y : gam.x, 2 * dt + (i >> 1));
}

// U = Ut - U (in place), Ut from the register operands.
template <typename T>
__device__ __forceinline__ void ut_minus(f32x4_t (&U)[4], const Raw8<T> (&ut)[2]) {
    float x[2][8];
    ut[0].get(x[0]);
    ut[1].get(x[1]);
#pragma unroll
    for (int R = 0; R < 2; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            U[2 * R][i] = x[R][i] - U[2 * R][i];
            U[2 * R + 1][i] = x[R][4 + i] - U[2 * R + 1][i];
        }
}

// One 1 KB direct-to-LDS copy: 16 bytes per lane from byte src + 16 l of the
// buffer (plus the wave-uniform soff) to dst + 16 l.  Kept out of the kernels'
// bodies: used there directly, the target builtin stops the host pass from
// emitting the kernel's launch stub.
__device__ __forceinline__ void dma_1k(__amdgpu_buffer_rsrc_t r, char *dst, unsigned src, unsigned soff, int l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, src + (unsigned)l * 16u, soff, 0, 0);
}

// Fragment f (in units of 512 elements) of an LDS operand slot, for lane l.
template <typename T>
__device__ __forceinline__ Frag<T> slot_frag(const char *slot, size_t elem, int l) {
    return *reinterpret_cast<const Frag<T> *>(slot + (elem + (size_t)l * 8) * sizeof(T));
}

// ============================================================================
// kda_segsum_kernel: a segment's state map.  Workgroup (segment g, head h):
// the state [L | Phi] of DV + DK columns starts at [0 | I] and runs through
// the segment's chunks, L with the Ut terms and Phi without.  Compute wave w
// owns 32 columns (two 16-column slabs): L's columns first, then Phi's.  The
// loader wave copies each chunk's W, Kh^T, Ut and decay into an LDS slot, one
// chunk ahead into the other slot when two fit.  A third slot (two chunks
// ahead) measured slower: one wave can hold at most 63 memory operations in
// flight, fewer than two chunks' copies, so the loader stalled at issue.  A
// sequence's last segment needs no summary; its workgroups return at once.
// ============================================================================
template <typename T, int DK, int DV>
struct SegsumPlan {
    static constexpr int ES = sizeof(T);
    static constexpr int NLW = DV / 32, NCW = (DV + DK) / 32;   // L waves, all compute waves
    static constexpr int THREADS = 64 * (NCW + 1);             // plus the loader
    static constexpr int W_B = 64 * DK * ES;                    // W, then Kh^T
    static constexpr int UG_SRC = (int)(Ws<T, DK, DV>::U * ES);  // Ut, then the decay (GAM_BYTE)
    static constexpr int UG_B = (int)round_up((size_t)64 * DV * ES + DK * 4, 1024);
    static constexpr int GAM_OFF = 2 * W_B + (int)(Ws<T, DK, DV>::GAM_BYTE - Ws<T, DK, DV>::U * ES);
    static constexpr int SLOT = 2 * W_B + UG_B;
    static constexpr int NOP = SLOT / 1024;
    // two slots when they fit (the loader one chunk ahead), else one
    static constexpr int NSLOT = 2 * SLOT <= kLdsMax ? 2 : 1;
    static constexpr int LDS_B = NSLOT * SLOT;
    static_assert(W_B % 1024 == 0 && UG_SRC % 1024 == 0 && LDS_B <= kLdsMax, "segment summary LDS plan");
    static_assert(THREADS <= kSegsumMaxThreads, "launch bound");
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kSegsumMaxThreads) void kda_segsum_kernel(KdaArgs a) {
    using P = SegsumPlan<T, DK, DV>;
    using WL = Ws<T, DK, DV>;
    using F = Frag<T>;
    constexpr int NKS = DK / 32, NDT = DK / 16, NSLOT = P::NSLOT;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int g = blk / a.H, h = blk % a.H;
    const int sq = seq_of_segment(a, g);
    const int p = g - seq_seg0(a, sq);
    if (g + 1 == seq_seg0(a, sq + 1)) return;   // the last segment of its sequence
    const int nch = seq_chk0(a, sq + 1) - seq_chk0(a, sq);
    const int slen = seq_seg_len(a, sq), n0 = p * slen, N = min(slen, nch - n0);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, col = l & 15, gq = l >> 4;
    const __amdgpu_buffer_rsrc_t wsr = seq_records<T, DK, DV>(a, sq, h);
    auto cbase = [&](int n) { return (unsigned)(n0 + n) * (unsigned)WL::BYTES; };

    if (wave == P::NCW) {
        // ---- loader: chunk n's W, Kh^T, Ut and decay into slot n % NSLOT ----
        auto issue_ops = [&](int n) {
            char *slot = lds + (n % NSLOT) * P::SLOT;
#pragma unroll
            for (int k = 0; k < P::NOP; ++k) {
                const int src = k < P::W_B / 1024       ? (int)(WL::W * P::ES) + k * 1024
                                : k < 2 * P::W_B / 1024 ? (int)(WL::KH * P::ES) + (k - P::W_B / 1024) * 1024
                                                        : P::UG_SRC + (k - 2 * P::W_B / 1024) * 1024;
                dma_1k(wsr, slot + k * 1024, (unsigned)src, cbase(n), l);
            }
        };
        if (NSLOT == 1) {
            issue_ops(0);
            wait_vm_all();
            lds_barrier();
#pragma unroll 1
            for (int n = 0; n < N; ++n) {
                lds_barrier();   // chunk n read
                if (n + 1 < N) issue_ops(n + 1);
                wait_vm_all();
                lds_barrier();
            }
            return;
        }
        // chunk n + 1 goes into the slot chunk n - 1 used, once every compute
        // wave has passed the barrier that ends chunk n - 1, and has landed
        // before the barrier that ends chunk n
        if (N > 0) issue_ops(0);
        wait_vm_all();
        lds_barrier();
#pragma unroll 1
        for (int n = 0; n < N; ++n) {
            if (n + 1 < N) issue_ops(n + 1);
            wait_vm_all();
            lds_barrier();
        }
        return;
    }

    // compute wave: matrix L (w < NLW) or Phi, slabs 2q and 2q + 1 of it
    const bool is_l = wave < P::NLW;
    const int q = is_l ? wave : wave - P::NLW;
    f32x4_t S[2][NDT];
    {
        // Phi starts at I: row 16 dt + 4g + i of column 32 q + 16 s2 + col
        const int diag = is_l ? -1 : 32 * q + col - 4 * gq;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[s2][dt][i] = 16 * dt + i == diag + 16 * s2 ? 1.f : 0.f;
    }
    lds_barrier();
#pragma unroll 1
    for (int n = 0; n < N; ++n) {
        const char *slot = lds + (n % NSLOT) * P::SLOT;
        const float2 gam = *reinterpret_cast<const float2 *>(
            slot + P::GAM_OFF + 4 * (gq * (DK / 4) + 2 * min(col, DK / 8 - 1)));
        // one slab after the other: U = Ut - W S (or -W S), S <- Diag(Gam) S + Kh^T U.
        // The fragments are read from LDS once per slab: one slab's temporaries
        // keep the wave within its registers at three waves per SIMD.
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            f32x4_t U[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) U[R] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const F b = tiles_to_frag<T>(S[s2][2 * ks], S[s2][2 * ks + 1]);
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    U[R] = mma(slot_frag<T>(slot, WL::W + (size_t)(R * NKS + ks) * 512, l), b, U[R]);
            }
            decay_rows<NDT>(S[s2], gam);
            if (is_l) {
                const char *ut = slot + 2 * P::W_B + ((size_t)(2 * q + s2) * 1024 + (size_t)l * 16) * sizeof(T);
                const Raw8<T> u8[2] = {*reinterpret_cast<const Raw8<T> *>(ut),
                                       *reinterpret_cast<const Raw8<T> *>(ut + 8 * sizeof(T))};
                ut_minus<T>(U, u8);
            } else {
#pragma unroll
                for (int R = 0; R < 4; ++R) U[R] = -U[R];
            }
            const F u[2] = {tiles_to_frag<T>(U[0], U[1]), tiles_to_frag<T>(U[2], U[3])};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    S[s2][dt] = mma(slot_frag<T>(slot + P::W_B, (size_t)(dt * 2 + kt) * 512, l), u[kt], S[s2][dt]);
        }
        if (NSLOT == 1) lds_barrier();   // chunk n read: the loader may refill the slot
        lds_barrier();
    }
    const SegRec<DK, DV> rec(a, h, g);
    if (is_l) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *reinterpret_cast<f32x4_t *>(rec.L + frag_off<DK>(2 * q + s2, dt, l)) = S[s2][dt];
    } else {
        // this lane's element (row 4g, column 32 q + col), formed here: hoisted above
        // the loop, the row offsets would take registers for its whole length
        int e0 = 4 * gq * DK + 32 * q + col;
        asm volatile("" : "+v"(e0));
        float *dst = rec.Phi + e0;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * dt + i) * DK + 16 * s2] = S[s2][dt][i];
    }
}

// ============================================================================
// kda_chain_kernel: the start state of every segment, in segment order.
// Workgroup (sequence, head, 16 state columns jt); wave ot computes the 16
// rows 16 ot .. 16 ot + 15 of S_start(p + 1) = Phi_p S_start(p) + L_p on the
// fp32 matrix cores.  The k index of the product runs over rows 16 dt + 4g + i
// for (dt, i) in turn, so lane group g's B operand is four consecutive rows
// of its column, one 16-byte read of the transposed LDS copy of the state.
// Each wave's rows of Phi_p and L_p are loaded into a ring of kChainAhead
// register sets, kChainAhead steps before their use: a step is one short
// product, far shorter than the memory latency.
// ============================================================================
constexpr int kChainAhead = 4;

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void kda_chain_kernel(KdaArgs a) {
    constexpr int NJT = DV / 16, NDT = DK / 16, SS = DK + 4;   // padded column of the LDS state copy
    __shared__ __attribute__((aligned(16))) float St[2][16][SS];   // St[.][col][row]
    // the NJT workgroups of one (sequence, head) read the same maps: kept on one
    // XCD, its L2 serves the maps to all of them
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int jt = blk % NJT, bh = blk / NJT;
    const int sq = bh / a.H, h = bh % a.H;
    const int ot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, col = l & 15, gq = l >> 4;
    const int sg0 = seq_seg0(a, sq), nseg = seq_seg0(a, sq + 1) - sg0;
    const int r0 = 16 * ot + 4 * gq;   // this lane's output rows r0 + i

    f32x4_t acc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = a.s0 ? a.s0[((size_t)bh * DK + r0 + i) * DV + 16 * jt + col] : 0.f;
    {
        const SegRec<DK, DV> rec(a, h, sg0);
        *reinterpret_cast<float4 *>(&St[0][col][r0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<f32x4_t *>(rec.S0 + frag_off<DK>(jt, ot, l)) = acc;
    }
    // ring of the maps of steps p .. p + kChainAhead - 1: Phi_p rows 16 ot + col at
    // columns 16 dt + 4g .. + 3, and L_p at this lane's outputs (nine 16-byte loads a
    // step: with the step's one store, the ring stays within the 63 memory
    // operations a wave can have in flight)
    float4 ph[kChainAhead][NDT];
    f32x4_t lp[kChainAhead];
    auto load_map = [&](int p, float4 (&phr)[NDT], f32x4_t &lpr) {
        const SegRec<DK, DV> rec(a, h, sg0 + p);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            phr[dt] = *reinterpret_cast<const float4 *>(rec.Phi + (16 * ot + col) * DK + 16 * dt + 4 * gq);
        lpr = *reinterpret_cast<const f32x4_t *>(rec.L + frag_off<DK>(jt, ot, l));
    };
    const int nsteps = nseg - 1;
    if (nsteps == 0) return;   // one segment: its start state is written
    // Straight-line steps: every step loads, computes, stores and meets the
    // barrier, whatever its index, so the memory-counter waits the compiler
    // places are exact (a conditional load or store makes it wait for all).
    // Steps past the last one repeat the last step: it reads the state it
    // read before (that LDS buffer is not rewritten) and stores the same values.
#pragma unroll
    for (int j = 0; j < kChainAhead; ++j) load_map(min(j, nsteps - 1), ph[j], lp[j]);
    lds_barrier();
    auto step = [&](int p, float4 (&phr)[NDT], f32x4_t &lpr) {
        const int cur = p & 1;
        // the whole column of the state first (one LDS wait), then the products
        // over four independent accumulators, summed at the end
        float4 b[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) b[dt] = *reinterpret_cast<const float4 *>(&St[cur][col][16 * dt + 4 * gq]);
        f32x4_t y4[4] = {lpr, zero4(), zero4(), zero4()};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            y4[0] = mma4(phr[dt].x, b[dt].x, y4[0]);
            y4[1] = mma4(phr[dt].y, b[dt].y, y4[1]);
            y4[2] = mma4(phr[dt].z, b[dt].z, y4[2]);
            y4[3] = mma4(phr[dt].w, b[dt].w, y4[3]);
        }
        const f32x4_t y = (y4[0] + y4[1]) + (y4[2] + y4[3]);
        load_map(min(p + kChainAhead, nsteps - 1), phr, lpr);
        const SegRec<DK, DV> rec(a, h, sg0 + p + 1);
        *reinterpret_cast<float4 *>(&St[cur ^ 1][col][r0]) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<f32x4_t *>(rec.S0 + frag_off<DK>(jt, ot, l)) = y;
        lds_barrier();
    };
#pragma unroll 1
    for (int p = 0; p < nsteps; p += kChainAhead) {
        // a repeated last step keeps the parity of the step it repeats
        const int last = nsteps - 1;
#pragma unroll
        for (int j = 0; j < kChainAhead; ++j) step(min(p + j, last), ph[j], lp[j]);
    }
}

// ============================================================================
// kda_segout_kernel: replay of one (segment, head) over all dv columns from its
// start state, writing o.  Compute waves 0 .. DV/16 - 1, then the store wave
// and the loader wave.
// With two operand slots (every bf16 shape) a chunk step has one barrier and
// the next chunk's loads fly under the current chunk's products; a shape whose
// operands only fit one slot (fp32) loads after computing, behind a second
// barrier.
// ============================================================================
template <typename T, int DK, int DV>
struct SegoutPlan {
    static constexpr int ES = sizeof(T);
    static constexpr int NCW = DV / 16;
    static constexpr int STORE_WAVE = NCW, LOAD_WAVE = NCW + 1;
    static constexpr int THREADS = 64 * (NCW + 2);
    static constexpr int OP_B = (int)(Ws<T, DK, DV>::U * ES);   // W, Qt, Kh^T, Bq: the record's first bytes
    static constexpr int NOP = OP_B / 1024;
    static constexpr int O_RB = DV * ES;                        // one token's output row
    static constexpr int O_STRIDE = O_RB + 16;
    static constexpr int O_B = 64 * O_STRIDE;
    static constexpr int NSLOT = (2 * OP_B + 2 * O_B <= kLdsMax) ? 2 : 1;
    static constexpr int LDS_B = NSLOT * (OP_B + O_B);
    static_assert(OP_B % 1024 == 0 && LDS_B <= kLdsMax, "segment replay LDS plan");
    static_assert(THREADS <= kSegoutMaxThreads, "launch bound");
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kSegoutMaxThreads) void kda_segout_kernel(KdaArgs a) {
    using P = SegoutPlan<T, DK, DV>;
    using WL = Ws<T, DK, DV>;
    using F = Frag<T>;
    constexpr int NKS = DK / 32, NDT = DK / 16, NSLOT = P::NSLOT;
    constexpr unsigned ES = sizeof(T);
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    auto op_slot = [&](int s) { return lds + s * P::OP_B; };
    auto o_slot = [&](int s) { return lds + NSLOT * P::OP_B + s * P::O_B; };

    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int g = blk / a.H, h = blk % a.H;
    const int sq = seq_of_segment(a, g);
    const int sg0 = seq_seg0(a, sq), p = g - sg0;
    const bool last_seg = g + 1 == seq_seg0(a, sq + 1);
    const int nch = seq_chk0(a, sq + 1) - seq_chk0(a, sq);
    const int slen = seq_seg_len(a, sq), n0 = p * slen, N = min(slen, nch - n0);
    const int tok0 = seq_tok0(a, sq), ntok = seq_tok0(a, sq + 1) - tok0;
    const int bh = sq * a.H + h;
    const bool chained = seq_seg0(a, a.B) > a.B;   // the chain wrote every segment's start state

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, col = l & 15, gq = l >> 4;
    const __amdgpu_buffer_rsrc_t wsr = seq_records<T, DK, DV>(a, sq, h);
    auto cbase = [&](int n) { return (unsigned)(n0 + n) * (unsigned)WL::BYTES; };

    if (wave == P::LOAD_WAVE) {
        // ---- loader: chunk n's W, Qt, Kh^T, Bq into its operand slot ----
        auto issue_ops = [&](int n) {
            char *slot = lds + (NSLOT == 2 ? (n & 1) : 0) * P::OP_B;
#pragma unroll
            for (int k = 0; k < P::NOP; ++k)
                dma_1k(wsr, slot + k * 1024, (unsigned)(k * 1024), cbase(n), l);
        };
        issue_ops(0);
        wait_vm_all();
        lds_barrier();
#pragma unroll 1
        for (int n = 0; n < N; ++n) {
            if (NSLOT == 2) {
                if (n + 1 < N) issue_ops(n + 1);
                wait_vm_all();
                lds_barrier();
            } else {
                lds_barrier();   // chunk n read
                if (n + 1 < N) issue_ops(n + 1);
                wait_vm_all();
                lds_barrier();
            }
        }
        if (NSLOT == 2) lds_barrier();   // the store wave's last step
    } else if (wave < P::NCW) {
        const int jt = wave;
        f32x4_t S[NDT];
        if (chained) {
            const float *s0 = SegRec<DK, DV>(a, h, g).S0;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) S[dt] = *reinterpret_cast<const f32x4_t *>(s0 + frag_off<DK>(jt, dt, l));
        } else {
            const float *s0 = a.s0 ? a.s0 + (size_t)bh * DK * DV : nullptr;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[dt][i] = s0 ? s0[(16 * dt + 4 * gq + i) * DV + 16 * jt + col] : 0.f;
        }
        ChunkRegs<T, DK, DV> cur, nxt;
        cur.load(wsr, cbase(0), jt, l, true);
        wait_vm_all();
        lds_barrier();
#pragma unroll 1
        for (int n = 0; n < N; ++n) {
            const int s = NSLOT == 2 ? (n & 1) : 0;
            const char *slot = op_slot(s);
            if (NSLOT == 2 && n + 1 < N) nxt.load(wsr, cbase(n + 1), jt, l, true);
            F Sb[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) Sb[ks] = tiles_to_frag<T>(S[2 * ks], S[2 * ks + 1]);
            // U = -W S and O = Qt S (O^T tiles: rows = value columns 4g + i, column = token)
            f32x4_t U[4], O[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) U[R] = O[R] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    U[R] = mma(slot_frag<T>(slot, WL::W + (size_t)(R * NKS + ks) * 512, l), Sb[ks], U[R]);
                    O[R] = mma(Sb[ks], slot_frag<T>(slot, WL::QT + (size_t)(R * NKS + ks) * 512, l), O[R]);
                }
            decay_rows<NDT>(S, cur.gam);
            ut_minus<T>(U, cur.ut);
            const F Ub[2] = {tiles_to_frag<T>(U[0], U[1]), tiles_to_frag<T>(U[2], U[3])};
            // O += Bq U, causal inside the chunk: token block R sees token k-steps kt <= R/2
#pragma unroll
            for (int R = 0; R < 4; ++R) O[R] = mma(Ub[0], slot_frag<T>(slot, WL::BT + (size_t)(R * 2) * 512, l), O[R]);
            O[2] = mma(Ub[1], slot_frag<T>(slot, WL::BT + (size_t)5 * 512, l), O[2]);
            O[3] = mma(Ub[1], slot_frag<T>(slot, WL::BT + (size_t)7 * 512, l), O[3]);
            // S <- Diag(Gam) S + Kh^T U
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    S[dt] = mma(slot_frag<T>(slot, WL::KH + (size_t)(dt * 2 + kt) * 512, l), Ub[kt], S[dt]);
            // stage O: lane (g, col) holds value columns 16 jt + 4g + i of token 16R + col
            char *os = o_slot(NSLOT == 2 ? (n & 1) : 0) + (16 * jt + 4 * gq) * ES;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                char *dst = os + (16 * R + col) * P::O_STRIDE;
                if (sizeof(T) == 2) {
                    *reinterpret_cast<uint2 *>(dst) =
                        make_uint2(pack_bf16x2(O[R][0], O[R][1]), pack_bf16x2(O[R][2], O[R][3]));
                } else {
                    *reinterpret_cast<float4 *>(dst) = make_float4(O[R][0], O[R][1], O[R][2], O[R][3]);
                }
            }
            if (NSLOT == 2) {
                wait_vm_all();   // the next chunk's registers have landed
                lds_barrier();   // and, after it, its operand slot
                cur = nxt;
            } else {
                lds_barrier();   // slot read, O staged
                if (n + 1 < N) cur.load(wsr, cbase(n + 1), jt, l, true);
                wait_vm_all();
                lds_barrier();
            }
        }
        if (NSLOT == 2) lds_barrier();   // the store wave's last step
        if (last_seg && a.sT) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.sT[((size_t)bh * DK + 16 * dt + 4 * gq + i) * DV + 16 * jt + col] = S[dt][i];
        }
    } else {
        // ---- store wave: o rows of one chunk from the staging buffer, 16 bytes per lane ----
        // o of this (sequence, head) as a raw buffer: token t at byte t * H * DV * ES, the
        // whole offset in the lane's offset so the range check drops rows past the end
        constexpr int LPR = P::O_RB / 16, RPI = 64 / LPR, NI = 64 / RPI;
        const unsigned orow = (unsigned)a.H * DV * ES;
        char *obase = static_cast<char *>(a.o) + ((size_t)tok0 * a.H + h) * DV * ES;
        const unsigned onum = (unsigned)ntok * orow - (unsigned)h * DV * ES;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(obase, 0, (int)onum, kBufWord3);
        const int lr = l / LPR, lc = l % LPR;
        auto store_chunk = [&](int n, const char *os) {
            u32x4_t v[NI];
#pragma unroll
            for (int r = 0; r < NI; ++r)
                v[r] = *reinterpret_cast<const u32x4_t *>(os + (r * RPI + lr) * P::O_STRIDE + lc * 16);
#pragma unroll
            for (int r = 0; r < NI; ++r) {
                const unsigned tok = (unsigned)((n0 + n) * 64 + r * RPI + lr);
                __builtin_amdgcn_raw_buffer_store_b128(v[r], orsrc, tok * orow + (unsigned)lc * 16, 0, 0);
            }
        };
        lds_barrier();
        if (NSLOT == 2) {
#pragma unroll 1
            for (int n = 0; n <= N; ++n) {
                if (n >= 1) store_chunk(n - 1, o_slot((n - 1) & 1));
                lds_barrier();
            }
        } else {
#pragma unroll 1
            for (int n = 0; n < N; ++n) {
                lds_barrier();
                store_chunk(n, o_slot(0));
                lds_barrier();
            }
        }
    }
}

// Dynamic LDS above 64 KB needs the kernel's attribute raised once per process.
hipError_t allow_lds(const void *kernel, int bytes, bool &done) {
    if (done || bytes <= 64 * 1024) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <typename T, int DK, int DV>
hipError_t launch_scan_typed(const KdaArgs &a, hipStream_t stream) {
    using PS = SegsumPlan<T, DK, DV>;
    using PO = SegoutPlan<T, DK, DV>;
    static bool sum_attr = false, out_attr = false;   // per process; setting twice is harmless
    const int total = seq_seg0(a, a.B);
    if (total > a.B) {
        hipError_t e = allow_lds((const void *)kda_segsum_kernel<T, DK, DV>, PS::LDS_B, sum_attr);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kda_segsum_kernel<T, DK, DV>), dim3(total * a.H), dim3(PS::THREADS), PS::LDS_B, stream,
                           a);
        hipLaunchKernelGGL((kda_chain_kernel<DK, DV>), dim3(a.B * a.H * (DV / 16)), dim3(64 * (DK / 16)), 0, stream,
                           a);
    }
    hipError_t e = allow_lds((const void *)kda_segout_kernel<T, DK, DV>, PO::LDS_B, out_attr);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_segout_kernel<T, DK, DV>), dim3(total * a.H), dim3(PO::THREADS), PO::LDS_B, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_scan(const KdaArgs &a, bool bf16, hipStream_t stream) {
    KDA_DISPATCH(launch_scan_typed)
}

}  // namespace kdaconv
