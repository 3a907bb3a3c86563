// Attention core of the MLA layers (Chimera pages, paper.rainbus.top,
// prerequisites section, the Multi-head Latent Attention paragraph): full,
// bidirectional softmax attention in which every head scores its queries
// against its own decompressed key part and one key part shared by all heads
// (K_direct):
//   s_ij = scale * (qn_i . kn_j + qd_i . kd_j),   o_i = sum_j softmax_j(s_ij) v_j
//
// One workgroup of four waves takes 128 queries of one (batch, head); each
// wave keeps 32 queries in its registers and walks the keys in tiles of 64
// with an online softmax (running maximum and sum per query), so the T x T
// scores never leave the chip.  Both products run on v_mfma_f32_16x16x32_bf16
// with every tile oriented so that a lane always holds one query:
//   S^T = K Q^T     (keys x queries; K from LDS, Q as register fragments)
//   O^T += V^T P^T  (values x queries; P straight from the S^T accumulators)
// so the softmax statistics, the rescaling of O and the final division stay
// inside a lane, and P needs no trip through LDS: the 8 k-slots a lane feeds
// to the second product are exactly the 8 keys its S^T accumulators hold, and
// the V^T fragments are read in that same key order.  The value tile is
// stored transposed in LDS ([dv][key]) so that each of those reads is two
// 8-byte runs.  The next key/value tile is loaded into registers while the
// current one's softmax and value product run.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace kdaconv {
namespace {

constexpr int kQW = 32;                 // queries per wave
constexpr int kCT = kQW / 16;           // 16-query column tiles per wave
constexpr int kQB = 4 * kQW;            // queries per workgroup
constexpr int kKT = 64;                 // keys per tile
constexpr int kDn = 128, kDr = 64, kDqk = kDn + kDr, kDv = 128;
constexpr int kKs = kDqk + 8;           // key-tile row stride in LDS (elements): 400 B, conflict-free 16 B reads
constexpr int kVs = kKT + 4;            // value-tile row stride in LDS (elements): 136 B, fewer bank conflicts
constexpr int kThreads = 256;
constexpr int kKnPer = kKT * (kDn / 8) / kThreads;   // 16-byte k_nope pieces of a key tile per thread
constexpr int kKdPer = kKT * (kDr / 8) / kThreads;   // 16-byte k_dir pieces
constexpr int kVPer = (kKT / 2) * (kDv / 8) / kThreads;   // (key pair, 8 value columns) tasks
static_assert(kKnPer == 4 && kKdPer == 2 && kVPer == 2, "tile loads split evenly over the workgroup");

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// x from lane (this lane ^ mask), through the LDS crossbar (no LDS memory)
__device__ __forceinline__ float xor_lanes(float x, int mask) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((__lane_id() ^ mask) << 2, __float_as_int(x)));
}
typedef Frag<bf16_t> BF;

struct Stage {
    u32x4_t kn[kKnPer], kd[kKdPer];
    u32x4_t v[kVPer][2];
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void mla_attention_kernel(
    MlaArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t Ks[kKT * kKs];   // [key][qk dims]
    __shared__ __attribute__((aligned(16))) bf16_t Vt[kDv * kVs];   // [value column][key]

    const int T = a.T, H = a.H;
    const int nqb = (T + kQB - 1) / kQB;
    // consecutive blocks of one XCD share a head, so its keys and values stay in that XCD's L2
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = blk % nqb, bh = blk / nqb, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c16 = l & 15,
              g = l >> 4;

    const bf16_t *qn = static_cast<const bf16_t *>(a.q_nope);
    const bf16_t *qd = static_cast<const bf16_t *>(a.q_dir);
    const bf16_t *kn = static_cast<const bf16_t *>(a.k_nope);
    const bf16_t *kd = static_cast<const bf16_t *>(a.k_dir);
    const bf16_t *vv = static_cast<const bf16_t *>(a.v);
    const size_t tok0 = (size_t)b * T;   // first token of this batch

    // Q^T fragments (B operand of S^T = K Q^T): column tile ct holds queries
    // q0 + 16ct + (l % 16); k-step s covers qk dims 32s .. 32s+31, lane group g
    // its dims 32s + 8g .. +7.  Queries past the end re-read the last one and
    // are never stored.
    const int q0 = qb * kQB + wave * kQW;
    BF qf[kCT][kDqk / 32];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
        const size_t q = tok0 + (size_t)min(q0 + 16 * ct + c16, T - 1);
        const bf16_t *pn = qn + (q * H + h) * kDn + 8 * g;
        const bf16_t *pd = qd + (q * H + h) * kDr + 8 * g;
#pragma unroll
        for (int s = 0; s < kDn / 32; ++s) qf[ct][s] = BF::ld8(pn + 32 * s);
#pragma unroll
        for (int s = 0; s < kDr / 32; ++s) qf[ct][kDn / 32 + s] = BF::ld8(pd + 32 * s);
    }

    // Tile loads through per-(batch, head) buffer resources whose range ends
    // at the last token of this batch's stream: keys past the end read zeros
    // (their scores are masked, their values then weigh nothing).  The tile's
    // first key enters as the uniform offset j0 * row bytes, so each lane's
    // offsets are fixed for the whole walk.  Thread t loads k_nope pieces
    // 4 (t % 4) .. +3 and k_dir pieces 2 (t % 4) .. +1 of key t / 4, and value
    // columns 8 (t / 32 + 8 i) .. +7 of keys 2 (t % 32) and 2 (t % 32) + 1,
    // stored transposed as packed key pairs.
    const unsigned rn = (unsigned)H * kDn * 2, rd = kDr * 2, rv = (unsigned)H * kDv * 2;   // row bytes
    const __amdgpu_buffer_rsrc_t kn_r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(kn + (tok0 * H + h) * kDn), 0, (int)((unsigned)(T - 1) * rn + kDn * 2), kBufWord3);
    const __amdgpu_buffer_rsrc_t kd_r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(kd + tok0 * kDr), 0, (int)((unsigned)T * rd), kBufWord3);
    const __amdgpu_buffer_rsrc_t v_r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(vv + (tok0 * H + h) * kDv), 0, (int)((unsigned)(T - 1) * rv + kDv * 2), kBufWord3);
    const int key = tid >> 2, q4 = tid & 3, m = tid & 31, cc = tid >> 5;
    const unsigned kn_off = (unsigned)key * rn + 64u * q4, kd_off = (unsigned)key * rd + 32u * q4;
    const unsigned v_off = (unsigned)(2 * m) * rv + 16u * cc;
    auto stage = [&](int j0, Stage &st) {
#pragma unroll
        for (int j = 0; j < kKnPer; ++j)
            st.kn[j] = __builtin_amdgcn_raw_buffer_load_b128(kn_r, kn_off + 16u * j, (unsigned)j0 * rn, 0);
#pragma unroll
        for (int j = 0; j < kKdPer; ++j)
            st.kd[j] = __builtin_amdgcn_raw_buffer_load_b128(kd_r, kd_off + 16u * j, (unsigned)j0 * rd, 0);
#pragma unroll
        for (int i = 0; i < kVPer; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                st.v[i][e] = __builtin_amdgcn_raw_buffer_load_b128(v_r, v_off + (unsigned)e * rv + 128u * i,
                                                                   (unsigned)j0 * rv, 0);
    };
    bf16_t *const kst = Ks + key * kKs;
    auto commit = [&](const Stage &st) {
#pragma unroll
        for (int j = 0; j < kKnPer; ++j) *reinterpret_cast<u32x4_t *>(kst + 32 * q4 + 8 * j) = st.kn[j];
#pragma unroll
        for (int j = 0; j < kKdPer; ++j) *reinterpret_cast<u32x4_t *>(kst + kDn + 16 * q4 + 8 * j) = st.kd[j];
#pragma unroll
        for (int i = 0; i < kVPer; ++i) {
            const u32x4_t lo = st.v[i][0], hi = st.v[i][1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // value columns c = 8 (cc + 8i) + 2w and c + 1 of keys 2m (low half) and 2m + 1
                uint32_t *d0 = reinterpret_cast<uint32_t *>(Vt + (8 * (cc + 8 * i) + 2 * w) * kVs + 2 * m);
                d0[0] = (lo[w] & 0xffffu) | (hi[w] << 16);
                d0[kVs / 2] = (lo[w] >> 16) | (hi[w] & 0xffff0000u);
            }
        }
    };

    f32x4_t O[kDv / 16][kCT];   // O^T: value rows 16rt + 4g + i of query column ct
#pragma unroll
    for (int rt = 0; rt < kDv / 16; ++rt)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) O[rt][ct] = zero4();
    float mrow[kCT], lsum[kCT];   // reference maximum of the raw scores; this lane's part of the sum
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
        mrow[ct] = -INFINITY;
        lsum[ct] = 0.f;
    }
    const float c = a.scale * 1.4426950408889634f;   // scores in log2 units

    Stage st;
    stage(0, st);
#pragma unroll 1
    for (int j0 = 0; j0 < T; j0 += kKT) {
        __syncthreads();   // every wave is done with the previous tile
        commit(st);
        __syncthreads();   // this tile is in LDS

        // S^T = K Q^T: key row tile rt (keys 16rt + 4g + i in lane l), query column tile ct
        f32x4_t S[4][kCT];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < kCT; ++ct) S[rt][ct] = zero4();
#pragma unroll
        for (int s = 0; s < kDqk / 32; ++s) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const BF kf = BF::ld8(Ks + (16 * rt + c16) * kKs + 32 * s + 8 * g);
#pragma unroll
                for (int ct = 0; ct < kCT; ++ct) S[rt][ct] = mma(kf, qf[ct][s], S[rt][ct]);
            }
            // at most one k-step of key fragments in flight: hoisting them all
            // would cost 96 registers
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next tile's loads run under the softmax and the second product
        // (issued here rather than earlier, which would keep 40 more registers
        // live through the first product)
        if (j0 + kKT < T) stage(j0 + kKT, st);
        __builtin_amdgcn_sched_barrier(0);
        if (j0 + kKT > T) {   // keys past the end of the stream weigh nothing
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (j0 + 16 * rt + 4 * g + i >= T)
#pragma unroll
                        for (int ct = 0; ct < kCT; ++ct) S[rt][ct][i] = -INFINITY;
        }
        BF pf[kCT][2];   // P^T fragments: query column ct, 32-key step ks
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
            // maximum over the tile's keys of this query (raw scores; scale > 0)
            float mx = -INFINITY;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[rt][ct][i]);
            // the four lane groups hold the other keys of the same query
            mx = fmaxf(mx, xor_lanes(mx, 16));
            mx = fmaxf(mx, xor_lanes(mx, 32));
            // The reference maximum moves only when some query's maximum grew
            // by more than 8 (log2 units): until then the weights 2^(s c - m c)
            // stay below 256 and the sums and O keep their common reference,
            // so the result is the same and O is rescaled far less often.
            const float mnew = fmaxf(mrow[ct], mx);
            if (__any((mnew - mrow[ct]) * c > 8.f)) {
                const float resc = __builtin_amdgcn_exp2f((mrow[ct] - mnew) * c);
                mrow[ct] = mnew;
                lsum[ct] *= resc;
#pragma unroll
                for (int rt = 0; rt < kDv / 16; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[rt][ct][i] *= resc;
            }
            const float mc = mrow[ct] * c;
            float x[4][4];
            float ps = 0.f;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[rt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rt][ct][i], c, -mc));
                    ps += x[rt][i];
                }
            lsum[ct] += ps;
            // k-slot (g, e) of step ks is key 32ks + 4g + e (e < 4) or 32ks + 16 + 4g + e - 4
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pf[ct][ks].v[e] = (bf16_t)x[2 * ks][e];
                    pf[ct][ks].v[4 + e] = (bf16_t)x[2 * ks + 1][e];
                }
        }
        // O^T += V^T P^T, V^T read in the same key order as the P^T slots
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int rt = 0; rt < kDv / 16; ++rt) {
                const bf16_t *row = Vt + (16 * rt + c16) * kVs + 32 * ks + 4 * g;
                const BF vf = BF::ld4x2(row, row + 16);
#pragma unroll
                for (int ct = 0; ct < kCT; ++ct) O[rt][ct] = mma(vf, pf[ct][ks], O[rt][ct]);
            }
        }
    }

    // o = O / (sum over the four lane groups' parts), in the input dtype.  The
    // lane's query and value columns are derived afresh from the lane id, so
    // that nothing lane-dependent has to stay live across the key walk.
    bf16_t *out = static_cast<bf16_t *>(a.o);
    int lo;   // the lane id, recomputed here (volatile: not merged with the one before the walk)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lo));
    const int co = lo & 15, go = lo >> 4;
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
        float z = lsum[ct];
        z += xor_lanes(z, 16);
        z += xor_lanes(z, 32);
        const float inv = 1.f / z;
        const int q = q0 + 16 * ct + co;
        if (q < T) {
            bf16_t *po = out + ((tok0 + (size_t)q) * H + h) * kDv + 4 * go;
#pragma unroll
            for (int rt = 0; rt < kDv / 16; ++rt) {
                const float r[4] = {O[rt][ct][0] * inv, O[rt][ct][1] * inv, O[rt][ct][2] * inv,
                                    O[rt][ct][3] * inv};
                st4<bf16_t>(po + 16 * rt, r);
            }
        }
    }
}

}  // namespace

hipError_t launch_mla_attention(const MlaArgs &a, hipStream_t stream) {
    const int nqb = (a.T + kQB - 1) / kQB;
    const int grid = a.B * a.H * nqb;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(mla_attention_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kdaconv
