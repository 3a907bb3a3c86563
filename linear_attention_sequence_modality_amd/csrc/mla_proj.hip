// The latent projections of multi-head latent attention (gfx950).
//
// Chimera pages (paper.rainbus.top, prerequisites section, the Multi-head
// Latent Attention paragraph): the hidden state is compressed into a
// low-dimensional latent, keys and values are decompressed from that latent,
// and one key part shared by every head (K_direct) is kept beside them.  With
// weights stored as a linear layer's [out, in]:
//   down:  c = x W_dkv^T  [rows, d_c]      k_dir  = x W_kr^T  [rows, d_dir]
//   up:    k_nope = c W_uk^T [rows, H d_nope]   v = c W_uv^T [rows, H dv]
// The attention over these is mla_attention_forward.
//
// Design.  Both steps are dense contractions, so they run on
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation, bf16 results).
// One kernel computes Y = X W^T for two weight/output pairs at once, output
// columns [0, N1) from (W1, Y1) and [N1, N1 + N2) from (W2, Y2), so the down
// step reads the hidden states once for the latent and K_direct, and the up
// step reads the latent once for keys and values.
//   * A 256-thread block computes a 256 x 64 tile; wave w owns rows 64w ..
//     64w + 63 (4 x 4 MFMA tiles).  X and W are both contiguous along the
//     contraction, so a lane's MFMA operand is 16 contiguous bytes of a row.
//   * The contraction advances 32 at a time through double-buffered LDS
//     (rows padded to 80 bytes against bank conflicts): the global loads of
//     step s+1 are in registers before the MFMAs of step s start and go to
//     the other buffer after them; one barrier per step.
//   * The tile leaves through LDS, so each lane stores 16 contiguous bytes.
//   * Block order: with a multiple of 8 column tiles (the decompression),
//     each XCD takes one eighth of them over every row slab, so its share of
//     W stays in its L2 and each slab of X is read once per XCD; otherwise
//     the column tiles of one slab are consecutive on one XCD, so the slab
//     comes from HBM once (the whole W is small there).
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace kdaconv {
namespace {

constexpr int PM = 256;           // rows per block
constexpr int PN = 64;            // columns per block
constexpr int PK = 32;            // contraction step
constexpr int PTHREADS = 256;
constexpr int PRS = PK + 8;       // LDS row stride in elements (80 bytes)
constexpr int A_EL = PM * PRS, B_EL = PN * PRS;
constexpr int OS = PN + 8;        // output staging row stride in elements
static_assert(2 * (A_EL + B_EL) >= PM * OS, "the output tile fits the operand buffers");

typedef Frag<bf16_t> BF;

__global__ __launch_bounds__(PTHREADS) __attribute__((amdgpu_waves_per_eu(3))) void mla_proj_kernel(
    MlaProjArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t sm[2 * (A_EL + B_EL)];
    const int n_tiles = (a.N1 + a.N2) / PN;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    int mt, nt;
    if (n_tiles % 8 == 0) {
        // eighths of the column tiles, one per XCD, each walked slab by slab:
        // an XCD keeps its eighth of W (n_tiles / 8 tiles of PN rows) in L2 and
        // reads each row slab of X once
        const int tg = n_tiles / 8, n_mt = gridDim.x / n_tiles;
        const int grp = blk / (n_mt * tg), rem = blk % (n_mt * tg);
        mt = rem / tg;
        nt = grp * tg + rem % tg;
    } else {
        // the column tiles of one slab together: the slab is read once from HBM
        mt = blk / n_tiles;
        nt = blk % n_tiles;
    }
    const int64_t m0 = (int64_t)mt * PM;
    const int n0 = nt * PN;
    const bool second = n0 >= a.N1;
    const bf16_t *W = static_cast<const bf16_t *>(second ? a.W2 : a.W1);
    bf16_t *Y = static_cast<bf16_t *>(second ? a.Y2 : a.Y1);
    const int nw = second ? n0 - a.N1 : n0;   // first column of the tile in its own output
    const int ldy = second ? a.N2 : a.N1;
    const int K = a.K;
    const bf16_t *X = static_cast<const bf16_t *>(a.X);
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;

    // staging map: thread t moves 16 bytes (8 elements) at chunk t % 4 of rows
    // t / 4 + 64 i of the X slab (rows past the end read the last row, and
    // their results are not stored) and of row t / 4 of the W tile
    const int lr = tid >> 2, lc = (tid & 3) * 8;
    const bf16_t *xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + lr + 64 * i < a.M ? m0 + lr + 64 * i : a.M - 1;
        xa[i] = X + row * K + lc;
    }
    const bf16_t *wb = W + (size_t)(nw + lr) * K + lc;
    uint4 ra0, ra1, ra2, ra3, rb;
#define KC_GLOAD(k0)                                                   \
    do {                                                               \
        ra0 = *reinterpret_cast<const uint4 *>(xa[0] + (k0));          \
        ra1 = *reinterpret_cast<const uint4 *>(xa[1] + (k0));          \
        ra2 = *reinterpret_cast<const uint4 *>(xa[2] + (k0));          \
        ra3 = *reinterpret_cast<const uint4 *>(xa[3] + (k0));          \
        rb = *reinterpret_cast<const uint4 *>(wb + (k0));              \
    } while (0)
#define KC_SSTORE(buf)                                                               \
    do {                                                                             \
        bf16_t *sa_ = sm + (buf) * (A_EL + B_EL), *sb_ = sa_ + A_EL;                 \
        *reinterpret_cast<uint4 *>(sa_ + lr * PRS + lc) = ra0;                       \
        *reinterpret_cast<uint4 *>(sa_ + (lr + 64) * PRS + lc) = ra1;                \
        *reinterpret_cast<uint4 *>(sa_ + (lr + 128) * PRS + lc) = ra2;               \
        *reinterpret_cast<uint4 *>(sa_ + (lr + 192) * PRS + lc) = ra3;               \
        *reinterpret_cast<uint4 *>(sb_ + lr * PRS + lc) = rb;                        \
    } while (0)

    f32x4_t acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = zero4();
    const int nk = K / PK;
    KC_GLOAD(0);
    KC_SSTORE(0);
    __syncthreads();
    const int fr = lane % 16, fk = 8 * (lane / 16);   // operand row (or column) and k offset of this lane
#pragma unroll 1
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if (s + 1 < nk) KC_GLOAD((s + 1) * PK);
        const bf16_t *sa = sm + buf * (A_EL + B_EL), *sb = sa + A_EL;
        BF fa[4], fb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) fa[r] = BF::ld8(sa + (64 * wave + 16 * r + fr) * PRS + fk);
#pragma unroll
        for (int c = 0; c < 4; ++c) fb[c] = BF::ld8(sb + (16 * c + fr) * PRS + fk);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = mma(fa[r], fb[c], acc[r][c]);
        // buffer buf ^ 1 was last read in step s - 1, before the previous barrier
        if (s + 1 < nk) KC_SSTORE(buf ^ 1);
        __syncthreads();
    }

#undef KC_GLOAD
#undef KC_SSTORE
    // the tile through LDS: lane l holds rows 4 (l / 16) + i of column l % 16 of each 16 x 16 tile
    bf16_t *so = sm;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                so[(64 * wave + 16 * r + 4 * (lane / 16) + i) * OS + 16 * c + fr] = (bf16_t)acc[r][c][i];
    __syncthreads();
    // 256 rows x 128 bytes: 8 chunks of 16 bytes per row, 8 per thread
#pragma unroll
    for (int j = 0; j < PM * PN / 8 / PTHREADS; ++j) {
        const int q = j * PTHREADS + tid, row = q / (PN / 8), ch = q % (PN / 8);
        if (m0 + row < a.M)
            *reinterpret_cast<uint4 *>(Y + (m0 + row) * ldy + nw + 8 * ch) =
                *reinterpret_cast<const uint4 *>(so + row * OS + 8 * ch);
    }
}

}  // namespace

hipError_t launch_mla_proj(const MlaProjArgs &a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    const int64_t blocks = (a.M + PM - 1) / PM * ((a.N1 + a.N2) / PN);
    hipLaunchKernelGGL(mla_proj_kernel, dim3((unsigned)blocks), dim3(PTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kdaconv
