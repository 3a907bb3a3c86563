// Modality-aware depthwise short convolution (gfx950).
//
// Chimera pages: the conv runs before every KDA update, separately per
// modality -- a causal 1D depthwise conv over text tokens and a depthwise 3D
// conv over the visual tokens on their (t, h, w) grid (rainbus "core method";
// genai-atlas "How it works").  Taps: text 4 (last tap on the current token),
// visual 3x3x3 with zero padding; time offset P = 1 (symmetric) or 2 (causal).
//
// Design.  A depthwise conv has no channel contraction, so there is no
// matrix-core work: 27 multiply-adds per output against 2 bytes in and 2 out.
// At the video stream's size the vector-ALU work (about 130 us) and the memory
// traffic (a copy of the same bytes takes about 160 us) are of one size, so
// the kernel keeps both lean and overlaps them.
//   * A 4-wave workgroup owns a tile of HR = 4 rows x WR = 8 w positions x 128
//     channels and marches over t.  For every input slice it stages the
//     (HR+2) x (WR+2) haloed tile in LDS with direct-to-LDS buffer loads of 16
//     bytes per lane (one instruction moves 4 positions of 256 bytes), double
//     buffered: the loads of slice t+1 fly while slice t is computed.  Tile
//     positions outside the grid are never loaded; their LDS bytes are zeroed
//     once, which is the conv's zero padding, so edge tiles run the same
//     branch-free window reads as interior ones.
//   * Wave w computes all 4 rows at positions w0 + 2w, w0 + 2w + 1; lane l
//     owns channels 2l, 2l+1.  It reads its 6 x 4 window of the slice from LDS
//     (one dword per position) and applies it to the three output slices
//     t-1, t, t+1 held in a 3-deep register ring whose slot index is static
//     after unrolling the march.  Taking all rows in one wave lets each
//     window row's byte permutes serve the three output rows that use it.
//   * bf16: taps are paired so that one v_dot2_f32_bf16 does two useful
//     multiply-adds: byte permutes form (x[w], x[w+1]) per channel for the
//     w-taps 0 and 1 of each row, and (x[row0], x[row1]) for w-tap 2 of rows 0
//     and 1; only w-tap 2 of row 2 uses a zero-padded weight pair.  The first
//     term of each output starts from an inline zero.  fp32 streams use fma.
//   * Output stores are issued before the next slice's loads, so the wait for
//     those loads mostly finds them done.
//   * Blocks run channel block by channel block, row group by row group, and
//     are remapped so each XCD works on a contiguous range of them: the halo
//     rows of neighbouring row groups are read by co-resident blocks.
//   * Single-slice grids (images) have nothing to march over in t: their
//     workgroups march down a column strip over row groups instead (below).
//   * Text tokens form a separate block range: a wave slides the 4-tap causal
//     window over TR consecutive text tokens.
#include "common.h"
#include "launch.h"

namespace kdaconv {
namespace {

constexpr int WR = 8;     // w positions per workgroup
constexpr int HR = 4;     // rows per workgroup
constexpr int JW = 2;     // w positions per wave (every wave computes all HR rows)
constexpr int TR = 16;    // text tokens per wave item
constexpr int NT = 256;   // threads per block (4 waves)
constexpr int LANES = 64;
constexpr int CPW = 2 * LANES;          // channels per workgroup
constexpr int TC = WR + 2;              // tile columns (w halo)
constexpr int TP = (HR + 2) * TC;       // tile positions per slice

typedef __attribute__((address_space(3))) void lds_void_t;

// Cache policy of the output stores: non-temporal (the nt bit of gfx9.4+ buffer stores), so
// the 400 MB output stream does not push the input halo rows that neighbouring tiles still
// read out of L2.
constexpr int kStoreNT = 2;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T> struct Ops;

template <> struct Ops<bf16_t> {
    typedef uint32_t XT;   // raw channel pair (c, c+1) of one token
    // taps of channels c (index 0) and c+1 (index 1), as bf16 pairs:
    //   pr[a][dh][ch] = (w[a][dh][0], w[a][dh][1])
    //   p2[a][ch]     = (w[a][0][2],  w[a][1][2])
    //   s2[a][ch]     = w[a][2][2] in channel ch's half of the pair, 0 in the other
    struct Taps {
        uint32_t pr[3][3][2], p2[3][2], s2[3][2];
    };
    // c0 (even, a valid channel) and c0+1 hold 54 consecutive taps = 27 dwords;
    // all are loaded at once, without conditions (!ok lanes zero them after)
    __device__ __forceinline__ static void load_taps(Taps &tp, const bf16_t *wv, int c0, bool ok) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(wv) + (size_t)c0 * 27 / 2;
        uint32_t d[27];
#pragma unroll
        for (int i = 0; i < 27; ++i) d[i] = p[i];
#pragma unroll
        for (int i = 0; i < 27; ++i) d[i] = ok ? d[i] : 0u;
        auto w = [&](int ch, int a, int dh, int e) -> uint32_t {
            const int i = ch * 27 + (a * 3 + dh) * 3 + e;
            return (i & 1) ? d[i >> 1] >> 16 : d[i >> 1] & 0xffffu;
        };
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
                for (int dh = 0; dh < 3; ++dh) tp.pr[a][dh][ch] = w(ch, a, dh, 0) | w(ch, a, dh, 1) << 16;
                tp.p2[a][ch] = w(ch, a, 0, 2) | w(ch, a, 1, 2) << 16;
                tp.s2[a][ch] = ch == 0 ? w(0, a, 2, 2) : w(1, a, 2, 2) << 16;
            }
    }
    __device__ __forceinline__ static XT lds_read(const char *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ __forceinline__ static XT zero() { return 0u; }
    __device__ __forceinline__ static float dot2(uint32_t x, uint32_t w, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, w), acc,
                                               false);
    }
    // dot2 onto a zero accumulator: the three-operand form with an inline 0
    // (the compiler otherwise zeroes a register for the two-operand form)
    __device__ __forceinline__ static float dot2_0(uint32_t x, uint32_t w) {
        float r;
        asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(w));
        return r;
    }
    __device__ __forceinline__ static void bstore(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                                  float a, float b) {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), r, voff, soff, kStoreNT);
    }
    __device__ __forceinline__ static XT load(const char *p) { return *reinterpret_cast<const uint32_t *>(p); }
    __device__ __forceinline__ static void store(char *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
    __device__ __forceinline__ static float lo(XT x) { return bf16_lo(x); }
    __device__ __forceinline__ static float hi(XT x) { return bf16_hi(x); }
    __device__ __forceinline__ static float tapw(const bf16_t *w, size_t i) { return (float)w[i]; }
};

template <> struct Ops<float> {
    typedef float2 XT;
    struct Taps {
        float w[27][2];
    };
    // channels c0 (a valid channel) and c0+1: 54 consecutive taps, loaded without conditions
    __device__ __forceinline__ static void load_taps(Taps &tp, const float *wv, int c0, bool ok) {
        const float *p = wv + (size_t)c0 * 27;
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            tp.w[tap][0] = p[tap];
            tp.w[tap][1] = p[27 + tap];
        }
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            tp.w[tap][0] = ok ? tp.w[tap][0] : 0.f;
            tp.w[tap][1] = ok ? tp.w[tap][1] : 0.f;
        }
    }
    __device__ __forceinline__ static XT lds_read(const char *p) { return *reinterpret_cast<const float2 *>(p); }
    __device__ __forceinline__ static XT zero() { return make_float2(0.f, 0.f); }
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static void bstore(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                                  float a, float b) {
        u32x2 u;
        u.x = __float_as_uint(a);
        u.y = __float_as_uint(b);
        __builtin_amdgcn_raw_buffer_store_b64(u, r, voff, soff, kStoreNT);
    }
    __device__ __forceinline__ static XT load(const char *p) { return *reinterpret_cast<const float2 *>(p); }
    __device__ __forceinline__ static void store(char *p, float a, float b) {
        *reinterpret_cast<float2 *>(p) = make_float2(a, b);
    }
    __device__ __forceinline__ static float lo(XT x) { return x.x; }
    __device__ __forceinline__ static float hi(XT x) { return x.y; }
    __device__ __forceinline__ static float tapw(const float *w, size_t i) { return w[i]; }
};

struct Layout {
    int n_cb[3];          // 128-channel blocks per stream
    int vis_blocks[3];    // B * n_cb * n_hg * n_wrun   (one per workgroup)
    int txt_items[3];     // B * n_trun * n_cb          (one per wave)
    int txt_blocks[3];
    int n_wrun, n_hg, n_trun;
    int n_gch;            // single-slice grids: runs of IG row groups
    int nblocks;
};

// One workgroup: (stream, batch, 128 channels, rows h0..h0+HR-1, w0..w0+WR-1), all t.
template <typename T, int PT, bool HIST>
struct VisualTile {
    typedef Ops<T> O;
    static constexpr int POS = CPW * (int)sizeof(T);      // bytes of one tile position
    static constexpr int LPP = POS / 16;                  // lanes per position in a 16-byte load
    static constexpr int PPI = LANES / LPP;               // positions per load instruction
    static constexpr int NI = TP / PPI;                   // load instructions per slice
    static constexpr int NIW = (NI + 3) / 4;              // per wave (at most)
    static_assert(TP % PPI == 0, "tile must split into whole load instructions");
    static constexpr int SLICE = TP * POS;                // LDS bytes per slice buffer

    __amdgpu_buffer_rsrc_t rx, ry, rh;   // input, output, history slices
    char *lds;            // two slice buffers
    int ti0;              // first input slice: -n_hist (history slices first)
    int wave, lane;
    int rowb, gt, gh, gw, h0, w0, wj;   // wj: first w position of this wave
    unsigned slice_bytes;  // one t-slice of the grid in the stream
    unsigned dma_off[NIW]; // lane's byte offset (t = 0) for each of its load instructions
    unsigned inb;          // bit i: load instruction i's position of this lane lies in the grid
    unsigned out_off;      // lane's byte offset (t = 0) of output (h0, wj)
    typename O::Taps taps;
    float acc[3][HR][JW][2];          // ring slot, row, position, channel
    typename O::XT x[HR + 2][JW + 2]; // the wave's window of the current slice

    // Positions outside the grid are never loaded: their 16 bytes of both slice
    // buffers hold zeros, written once before the march (the zero padding).
    template <bool EDGE>
    __device__ __forceinline__ void zero_outside() {
        if (!EDGE) return;
#pragma unroll
        for (int i = 0; i < NIW; ++i) {
            const int k = wave + 4 * i;
            if (k < NI && !(inb >> i & 1u))
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    *reinterpret_cast<u32x4_t *>(lds + b * SLICE + k * 1024 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    // mask: bit i set if load instruction i is issued for this lane
    __device__ __forceinline__ void issue_slice(int ti, unsigned mask) {
        char *buf = lds + (ti & 1) * SLICE;
        // history slice ti < 0 sits at slice ti - ti0 of the history buffer
        // (which has no text tokens: the segment has none either)
        const bool hist = HIST && ti < 0;
        const unsigned soff = (unsigned)(hist ? ti - ti0 : ti) * slice_bytes;
#pragma unroll
        for (int i = 0; i < NIW; ++i) {
            const int k = wave + 4 * i;
            if (k < NI && (mask >> i & 1u))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(hist ? rh : rx, (lds_void_t *)(buf + k * 1024), 16,
                                                         dma_off[i], soff, 0, 0);
        }
    }

    __device__ __forceinline__ void read_window(int ti) {
        const char *buf = lds + (ti & 1) * SLICE + lane * (int)(POS / LANES) + JW * wave * POS;
#pragma unroll
        for (int r = 0; r < HR + 2; ++r)
#pragma unroll
            for (int c = 0; c < JW + 2; ++c) x[r][c] = O::lds_read(buf + (r * TC + c) * POS);
    }

    template <int P, bool EDGE>
    __device__ __forceinline__ void flush(int t_done, bool active) {
        constexpr int slot = ((P + PT) % 3 + 3) % 3;   // slot of output slice ti + PT - 3
        if (active && t_done >= 0 && t_done < gt) {
            const unsigned soff = (unsigned)t_done * slice_bytes;
#pragma unroll
            for (int r = 0; r < HR; ++r)
#pragma unroll
                for (int j = 0; j < JW; ++j)
                    if (!EDGE || (h0 + r < gh && wj + j < gw))
                        O::bstore(ry, out_off + (unsigned)((r * gw + j) * rowb), soff, acc[slot][r][j][0],
                                  acc[slot][r][j][1]);
        }
    }

    // Input slice ti (ti = P mod 6) into the three output slices it feeds.  The
    // window rows rr are taken in order, so each accumulator still receives its
    // taps in the order dh = 0, 1, 2 (then, for bf16, the paired and the single
    // w-tap 2 terms): the window row rr is row dh = rr - r of output row r.
    template <int P>
    __device__ __forceinline__ void compute() {
        constexpr int SL[3] = {((P + PT) % 3 + 3) % 3, ((P + PT - 1) % 3 + 3) % 3, ((P + PT - 2) % 3 + 3) % 3};
#pragma unroll
        for (int rr = 0; rr < HR + 2; ++rr)
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                if constexpr (sizeof(T) == 2) {
                    const uint32_t plo = __builtin_amdgcn_perm(x[rr][j + 1], x[rr][j], 0x05040100u);
                    const uint32_t phi = __builtin_amdgcn_perm(x[rr][j + 1], x[rr][j], 0x07060302u);
#pragma unroll
                    for (int dh = 0; dh < 3; ++dh) {
                        const int r = rr - dh;
                        if (r < 0 || r >= HR) continue;
#pragma unroll
                        for (int a = 0; a < 3; ++a) {
                            float &c0 = acc[SL[a]][r][j][0], &c1 = acc[SL[a]][r][j][1];
                            if (a == 0 && dh == 0) {   // first term of output slice ti + PT
                                c0 = O::dot2_0(plo, taps.pr[a][dh][0]);
                                c1 = O::dot2_0(phi, taps.pr[a][dh][1]);
                            } else {
                                c0 = O::dot2(plo, taps.pr[a][dh][0], c0);
                                c1 = O::dot2(phi, taps.pr[a][dh][1], c1);
                            }
                        }
                    }
                    if (rr >= 2) {
                        const int r = rr - 2;
                        const uint32_t qlo = __builtin_amdgcn_perm(x[r + 1][j + 2], x[r][j + 2], 0x05040100u);
                        const uint32_t qhi = __builtin_amdgcn_perm(x[r + 1][j + 2], x[r][j + 2], 0x07060302u);
#pragma unroll
                        for (int a = 0; a < 3; ++a) {
                            float &c0 = acc[SL[a]][r][j][0], &c1 = acc[SL[a]][r][j][1];
                            c0 = O::dot2(qlo, taps.p2[a][0], c0);
                            c1 = O::dot2(qhi, taps.p2[a][1], c1);
                            c0 = O::dot2(x[rr][j + 2], taps.s2[a][0], c0);
                            c1 = O::dot2(x[rr][j + 2], taps.s2[a][1], c1);
                        }
                    }
                } else {
#pragma unroll
                    for (int dh = 0; dh < 3; ++dh) {
                        const int r = rr - dh;
                        if (r < 0 || r >= HR) continue;
#pragma unroll
                        for (int a = 0; a < 3; ++a)
#pragma unroll
                            for (int e = 0; e < 3; ++e) {
                                const int tap = (a * 3 + dh) * 3 + e;
                                float &c0 = acc[SL[a]][r][j][0], &c1 = acc[SL[a]][r][j][1];
                                const bool fresh = tap == 0;   // first term of output slice ti + PT
                                c0 = __builtin_fmaf(taps.w[tap][0], x[rr][j + e].x, fresh ? 0.f : c0);
                                c1 = __builtin_fmaf(taps.w[tap][1], x[rr][j + e].y, fresh ? 0.f : c1);
                            }
                    }
                }
            }
    }

    // Step P of the march (ti = 6m + P).  Input slice ti contributes tap
    // slice a to output slice ti + PT - a, kept in ring slot (P + PT - a) mod 3.
    template <int P, bool EDGE>
    __device__ __forceinline__ void step(int ti, bool active) {
        const bool live = (!HIST || ti >= ti0) && ti < gt;   // steps before ti0 only align the march
        // Slice ti has landed once every wave's direct-to-LDS loads of it have
        // retired: wait for them explicitly (the compiler does not track them
        // across the loop back-edge), then meet at the barrier, which also ends
        // every read of slice ti-1.  The wait covers this wave's output stores
        // of the previous step too; they are issued before the slice loads, so
        // they are mostly done by the time the loads are.
        if (live) {
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            lds_barrier();
            read_window(ti);
        }
        flush<P, EDGE>(ti + PT - 3, active);
        if (live && ti + 1 < gt) issue_slice(ti + 1, EDGE ? inb : ~0u);
        if (live && active) compute<P>();
    }

    template <bool EDGE>
    __device__ void march(bool active) {
        zero_outside<EDGE>();
        issue_slice(HIST ? ti0 : 0, EDGE ? inb : ~0u);
        // empty steps past the last slice flush the last output slices; with
        // history the march starts at -6 so that step<P> still sees ti = P mod 6
        const int last = gt + 2 - PT;
#pragma unroll 1
        for (int ti = HIST ? -6 : 0; ti <= last; ti += 6) {
            step<0, EDGE>(ti, active);
            if (ti + 1 > last) break;
            step<1, EDGE>(ti + 1, active);
            if (ti + 2 > last) break;
            step<2, EDGE>(ti + 2, active);
            if (ti + 3 > last) break;
            step<3, EDGE>(ti + 3, active);
            if (ti + 4 > last) break;
            step<4, EDGE>(ti + 4, active);
            if (ti + 5 > last) break;
            step<5, EDGE>(ti + 5, active);
        }
    }
};

template <typename T, int PT, bool HIST>
__device__ void visual_block(const ConvArgs &a, const Layout &L, int s, int blk, int wave, int lane, char *lds) {
    typedef VisualTile<T, PT, HIST> V;
    // channel block outermost, then row groups, then w-runs
    const int wrun = blk % L.n_wrun;
    int rest = blk / L.n_wrun;
    const int hg = rest % L.n_hg;
    rest /= L.n_hg;
    const int cb = rest % L.n_cb[s];
    const int b = rest / L.n_cb[s];
    const int C = a.C[s];
    const int c0 = cb * CPW + 2 * lane;
    const bool ok = c0 < C;   // lanes past the last channel compute zeros and store nothing

    V v;
    v.wave = wave;
    v.lane = lane;
    v.lds = lds;
    v.rowb = C * (int)sizeof(T);
    v.gt = a.gt;
    v.gh = a.gh;
    v.gw = a.gw;
    v.h0 = hg * HR;
    v.w0 = wrun * WR;
    v.wj = v.w0 + JW * wave;
    v.slice_bytes = (unsigned)(a.gh * a.gw) * (unsigned)v.rowb;
    const size_t bbytes = (size_t)a.T * v.rowb;   // < 4 GiB, checked on the host
    v.rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.x[s])) + (size_t)b * bbytes, 0, (int)(unsigned)bbytes,
        kBufWord3);
    v.ry = __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(a.y[s]) + (size_t)b * bbytes, 0,
                                             (int)(unsigned)bbytes, kBufWord3);
    if constexpr (HIST) {
        v.ti0 = -a.n_hist;
        const size_t hbytes = (size_t)a.n_hist * v.slice_bytes;   // history of one batch
        v.rh = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(static_cast<const char *>(a.hx[s])) + (size_t)b * hbytes, 0, (int)(unsigned)hbytes,
            kBufWord3);
    }
    // tile position p of load instruction k: k * PPI + lane / LPP; positions
    // outside the grid are not loaded (their offsets are clamped into the grid
    // all the same)
    const unsigned chan = (unsigned)(cb * V::POS) + (unsigned)(lane % V::LPP) * 16u;
    v.inb = 0u;
#pragma unroll
    for (int i = 0; i < V::NIW; ++i) {
        const int k = wave + 4 * i;
        const int p = k * V::PPI + lane / V::LPP;
        const int hu = v.h0 - 1 + p / TC, wu = v.w0 - 1 + p % TC;
        const int hh = min(max(hu, 0), a.gh - 1);
        const int ww = min(max(wu, 0), a.gw - 1);
        v.dma_off[i] = (unsigned)(a.n_text + hh * a.gw + ww) * (unsigned)v.rowb + chan;
        if (hu == hh && wu == ww) v.inb |= 1u << i;
    }
    v.out_off = (unsigned)(a.n_text + v.h0 * a.gw + v.wj) * (unsigned)v.rowb + (unsigned)((ok ? c0 : 0) * (int)sizeof(T));
    Ops<T>::load_taps(v.taps, static_cast<const T *>(a.wv[s]), ok ? c0 : 0, ok);
#pragma unroll
    for (int sl = 0; sl < 3; ++sl)
#pragma unroll
        for (int r = 0; r < HR; ++r)
#pragma unroll
            for (int j = 0; j < JW; ++j) v.acc[sl][r][j][0] = v.acc[sl][r][j][1] = 0.f;
    // every wave takes part in the loads and barriers; waves whose positions
    // all lie past the grid and lanes past the last channel compute nothing and
    // store nothing
    const bool active = ok && v.wj < a.gw;
    if (v.h0 >= 1 && v.h0 + HR < a.gh && v.w0 >= 1 && v.w0 + WR < a.gw)
        v.template march<false>(active);
    else
        v.template march<true>(active);
}

// ---- single-slice grids (images: grid_t = 1) ------------------------------------
// With one latent slice only the centre time taps (slice PT of the three) see
// data, and there is nothing to march over in t.  A workgroup instead owns a
// column strip (8 w positions x 128 channels) of IG consecutive row groups of
// 4 rows and marches down it: step g stages the haloed 6 x 10 tile of row
// group g (double buffered, the loads of group g+1 in flight under the
// compute of group g), computes its 4 x 8 outputs from that tile alone and
// stores them a step later.  Tile positions outside the grid (the image's
// border, which moves with the row group at the top and bottom) are written
// as zeros into the tile by the lane that would have loaded them.
constexpr int IG = 8;   // row groups per workgroup

template <typename T, int PT>
struct ImageTile {
    typedef Ops<T> O;
    static constexpr int POS = CPW * (int)sizeof(T);
    static constexpr int LPP = POS / 16;
    static constexpr int PPI = LANES / LPP;
    static constexpr int NI = TP / PPI;
    static constexpr int NIW = (NI + 3) / 4;
    static constexpr int SLICE = TP * POS;
    static constexpr int AC = PT;   // the time tap slice that meets the single input slice

    __amdgpu_buffer_rsrc_t rx, ry;
    char *lds;
    int wave, lane, rowb, gh, gw, w0, wj, n_hg, g0;
    unsigned group_bytes;   // one row group of the grid in the stream
    unsigned base_off[NIW]; // lane's byte offset of its load instructions' positions for row group 0 (mod 2^32)
    int prow[NIW], pcol[NIW];   // tile row and column of those positions
    unsigned out_off;     // lane's byte offset of output (row 0, wj)
    typename O::Taps taps;
    float acc[2][HR][JW][2];
    typename O::XT x[HR + 2][JW + 2];

    __device__ __forceinline__ void issue(int g) {   // row group g (absolute) into buffer g & 1
        char *buf = lds + (g & 1) * SLICE;
#pragma unroll
        for (int i = 0; i < NIW; ++i) {
            const int k = wave + 4 * i;
            if (k >= NI) continue;
            const int hu = HR * g - 1 + prow[i], wu = w0 - 1 + pcol[i];
            if (hu >= 0 && hu < gh && wu >= 0 && wu < gw)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(buf + k * 1024), 16,
                                                         base_off[i] + (unsigned)g * group_bytes, 0, 0, 0);
            else
                *reinterpret_cast<u32x4_t *>(buf + k * 1024 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    __device__ __forceinline__ void read_window(int g) {
        const char *buf = lds + (g & 1) * SLICE + lane * (int)(POS / LANES) + JW * wave * POS;
#pragma unroll
        for (int r = 0; r < HR + 2; ++r)
#pragma unroll
            for (int c = 0; c < JW + 2; ++c) x[r][c] = O::lds_read(buf + (r * TC + c) * POS);
    }

    template <int SLOT>
    __device__ __forceinline__ void flush(int g, bool active) {   // outputs of row group g
        if (!active || g < g0 || g >= n_hg) return;
        const unsigned goff = (unsigned)g * group_bytes;
#pragma unroll
        for (int r = 0; r < HR; ++r)
#pragma unroll
            for (int j = 0; j < JW; ++j)
                if (HR * g + r < gh && wj + j < gw)
                    O::bstore(ry, out_off + goff + (unsigned)((r * gw + j) * rowb), 0u, acc[SLOT][r][j][0],
                              acc[SLOT][r][j][1]);
    }

    // tap slice AC of the window into slot SLOT, every accumulator fresh; the
    // per-accumulator order of terms is that of the slice marches
    template <int SLOT>
    __device__ __forceinline__ void compute() {
#pragma unroll
        for (int rr = 0; rr < HR + 2; ++rr)
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                if constexpr (sizeof(T) == 2) {
                    const uint32_t plo = __builtin_amdgcn_perm(x[rr][j + 1], x[rr][j], 0x05040100u);
                    const uint32_t phi = __builtin_amdgcn_perm(x[rr][j + 1], x[rr][j], 0x07060302u);
#pragma unroll
                    for (int dh = 0; dh < 3; ++dh) {
                        const int r = rr - dh;
                        if (r < 0 || r >= HR) continue;
                        float &c0 = acc[SLOT][r][j][0], &c1 = acc[SLOT][r][j][1];
                        if (dh == 0) {
                            c0 = O::dot2_0(plo, taps.pr[AC][0][0]);
                            c1 = O::dot2_0(phi, taps.pr[AC][0][1]);
                        } else {
                            c0 = O::dot2(plo, taps.pr[AC][dh][0], c0);
                            c1 = O::dot2(phi, taps.pr[AC][dh][1], c1);
                        }
                    }
                    if (rr >= 2) {
                        const int r = rr - 2;
                        const uint32_t qlo = __builtin_amdgcn_perm(x[r + 1][j + 2], x[r][j + 2], 0x05040100u);
                        const uint32_t qhi = __builtin_amdgcn_perm(x[r + 1][j + 2], x[r][j + 2], 0x07060302u);
                        float &c0 = acc[SLOT][r][j][0], &c1 = acc[SLOT][r][j][1];
                        c0 = O::dot2(qlo, taps.p2[AC][0], c0);
                        c1 = O::dot2(qhi, taps.p2[AC][1], c1);
                        c0 = O::dot2(x[rr][j + 2], taps.s2[AC][0], c0);
                        c1 = O::dot2(x[rr][j + 2], taps.s2[AC][1], c1);
                    }
                } else {
#pragma unroll
                    for (int dh = 0; dh < 3; ++dh) {
                        const int r = rr - dh;
                        if (r < 0 || r >= HR) continue;
#pragma unroll
                        for (int e = 0; e < 3; ++e) {
                            const int tap = (AC * 3 + dh) * 3 + e;
                            float &c0 = acc[SLOT][r][j][0], &c1 = acc[SLOT][r][j][1];
                            const bool fresh = dh == 0 && e == 0;
                            c0 = __builtin_fmaf(taps.w[tap][0], x[rr][j + e].x, fresh ? 0.f : c0);
                            c1 = __builtin_fmaf(taps.w[tap][1], x[rr][j + e].y, fresh ? 0.f : c1);
                        }
                    }
                }
            }
    }

    template <int SLOT>
    __device__ __forceinline__ void step(int g, bool active) {
        const int g1 = min(g0 + IG, n_hg);
        if (g < g1) {
            // row group g has landed once every wave's loads of it have retired;
            // the barrier also ends every read of group g - 1's buffer
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
            lds_barrier();
            read_window(g);
        }
        flush<SLOT ^ 1>(g - 1, active);
        if (g + 1 < g1) issue(g + 1);
        if (g < g1 && active) compute<SLOT>();
    }

    __device__ void march(bool active) {
        issue(g0);
        const int g1 = min(g0 + IG, n_hg);
#pragma unroll 1
        for (int g = g0; g <= g1; g += 2) {   // one step past the last group stores it
            step<0>(g, active);
            if (g + 1 > g1) break;
            step<1>(g + 1, active);
        }
    }
};

template <typename T, int PT>
__device__ void image_block(const ConvArgs &a, const Layout &L, int s, int blk, int wave, int lane, char *lds) {
    typedef ImageTile<T, PT> V;
    // channel block outermost, then row-group runs, then w-runs
    const int wrun = blk % L.n_wrun;
    int rest = blk / L.n_wrun;
    const int gch = rest % L.n_gch;
    rest /= L.n_gch;
    const int cb = rest % L.n_cb[s];
    const int b = rest / L.n_cb[s];
    const int C = a.C[s];
    const int c0 = cb * CPW + 2 * lane;
    const bool ok = c0 < C;

    V v;
    v.wave = wave;
    v.lane = lane;
    v.lds = lds;
    v.rowb = C * (int)sizeof(T);
    v.gh = a.gh;
    v.gw = a.gw;
    v.w0 = wrun * WR;
    v.wj = v.w0 + JW * wave;
    v.n_hg = L.n_hg;
    v.g0 = gch * IG;
    v.group_bytes = (unsigned)(HR * a.gw) * (unsigned)v.rowb;
    const size_t bbytes = (size_t)a.T * v.rowb;   // < 4 GiB, checked on the host
    v.rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(a.x[s])) + (size_t)b * bbytes, 0, (int)(unsigned)bbytes,
        kBufWord3);
    v.ry = __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(a.y[s]) + (size_t)b * bbytes, 0,
                                             (int)(unsigned)bbytes, kBufWord3);
    const int chan = cb * V::POS + (lane % V::LPP) * 16;
#pragma unroll
    for (int i = 0; i < V::NIW; ++i) {
        const int k = wave + 4 * i;
        const int p = k * V::PPI + lane / V::LPP;
        v.prow[i] = p / TC;
        v.pcol[i] = p % TC;
        // row group 0's position (row prow - 1, column w0 - 1 + pcol), modulo 2^32:
        // "negative" for the halo row above the image, which row group 0 never
        // loads; adding g row groups gives the true offset wherever one is loaded
        v.base_off[i] = (unsigned)(a.n_text + (v.prow[i] - 1) * a.gw + v.w0 - 1 + v.pcol[i]) * (unsigned)v.rowb +
                        (unsigned)chan;
    }
    v.out_off = (unsigned)(a.n_text + v.wj) * (unsigned)v.rowb + (unsigned)((ok ? c0 : 0) * (int)sizeof(T));
    Ops<T>::load_taps(v.taps, static_cast<const T *>(a.wv[s]), ok ? c0 : 0, ok);
    v.march(ok && v.wj < a.gw);
}

template <typename T>
__device__ void text_item(const ConvArgs &a, const Layout &L, int s, int item, int lane) {
    typedef Ops<T> O;
    const int n_cb = L.n_cb[s];
    const int cb = item % n_cb;
    const int rest = item / n_cb;
    const int trun = rest % L.n_trun;
    const int b = rest / L.n_trun;
    const int C = a.C[s];
    const int c0 = cb * CPW + 2 * lane;
    if (c0 >= C) return;
    const int rowb = C * (int)sizeof(T);
    const char *x = static_cast<const char *>(a.x[s]) + (size_t)b * a.T * rowb + c0 * sizeof(T);
    char *y = static_cast<char *>(a.y[s]) + (size_t)b * a.T * rowb + c0 * sizeof(T);
    const T *wt = static_cast<const T *>(a.wt[s]);
    float w[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j][0] = O::tapw(wt, (size_t)c0 * 4 + j);
        w[j][1] = O::tapw(wt, (size_t)(c0 + 1) * 4 + j);
    }
    const int i0 = trun * TR;
    float xin[TR + 3][2];
    // all TR + 3 loads at once from clamped (valid) tokens; tokens outside the
    // text are zero (the causal padding, and the end of the text)
    typename O::XT raw[TR + 3];
#pragma unroll
    for (int m = 0; m < TR + 3; ++m) raw[m] = O::load(x + (size_t)min(max(i0 - 3 + m, 0), a.n_text - 1) * rowb);
#pragma unroll
    for (int m = 0; m < TR + 3; ++m) {
        const int src = i0 - 3 + m;
        const bool in = src >= 0 && src < a.n_text;
        xin[m][0] = in ? O::lo(raw[m]) : 0.f;
        xin[m][1] = in ? O::hi(raw[m]) : 0.f;
    }
#pragma unroll
    for (int m = 0; m < TR; ++m) {
        const int i = i0 + m;
        if (i < a.n_text) {
            float o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o0 = __builtin_fmaf(w[j][0], xin[m + j][0], o0);
                o1 = __builtin_fmaf(w[j][1], xin[m + j][1], o1);
            }
            O::store(y + (size_t)i * rowb, o0, o1);
        }
    }
}

// bf16: at most 128 VGPRs, so four 4-wave blocks share a CU (LDS: 4 x 30 KB).
// IMG: the single-slice grid variant (grid_t = 1, no history).
template <typename T, int PT, bool HIST, bool IMG>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 2 : 4))) void conv_kernel(
    ConvArgs a, Layout L) {
    __shared__ __attribute__((aligned(1024))) char lds[2 * VisualTile<T, PT, HIST>::SLICE];
    int blk = xcd_remap(blockIdx.x, L.nblocks);
    const int wave = uniform(threadIdx.x / LANES), lane = threadIdx.x % LANES;
    constexpr int WPB = NT / LANES;
#pragma unroll 1
    for (int s = 0; s < 3; ++s) {
        if (blk < L.vis_blocks[s]) {
            if constexpr (IMG)
                image_block<T, PT>(a, L, s, blk, wave, lane, lds);
            else
                visual_block<T, PT, HIST>(a, L, s, blk, wave, lane, lds);
            return;
        }
        blk -= L.vis_blocks[s];
        if (blk < L.txt_blocks[s]) {
            const int item = uniform(blk * WPB + wave);
            if (item < L.txt_items[s]) text_item<T>(a, L, s, item, lane);
            return;
        }
        blk -= L.txt_blocks[s];
    }
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, bool bf16, hipStream_t stream) {
    constexpr int WPB = NT / LANES;
    // history slices exist only for time-causal segments; a separate
    // instantiation keeps the extra buffer resource out of the other kernels
    const bool hist = a.causal_t && a.n_hist > 0;
    const bool img = a.gt == 1 && !hist;   // one latent slice: march down the rows instead
    Layout L;
    L.n_wrun = (a.gw + WR - 1) / WR;
    L.n_hg = (a.gh + HR - 1) / HR;
    L.n_gch = (L.n_hg + IG - 1) / IG;
    L.n_trun = (a.n_text + TR - 1) / TR;
    const int n_vis = a.gt * a.gh * a.gw;
    L.nblocks = 0;
    for (int s = 0; s < 3; ++s) {
        L.n_cb[s] = (a.C[s] + CPW - 1) / CPW;
        L.vis_blocks[s] = n_vis ? a.B * L.n_cb[s] * (img ? L.n_gch : L.n_hg) * L.n_wrun : 0;
        L.txt_items[s] = a.B * L.n_trun * L.n_cb[s];
        L.txt_blocks[s] = (L.txt_items[s] + WPB - 1) / WPB;
        L.nblocks += L.vis_blocks[s] + L.txt_blocks[s];
    }
    if (L.nblocks == 0) return hipSuccess;
#define KC_LAUNCH(TT, PTT, HISTT, IMGT) \
    hipLaunchKernelGGL((conv_kernel<TT, PTT, HISTT, IMGT>), dim3(L.nblocks), dim3(NT), 0, stream, a, L)
    if (bf16) {
        if (hist)
            KC_LAUNCH(bf16_t, 2, true, false);
        else if (a.causal_t)
            {
            if (img)
                KC_LAUNCH(bf16_t, 2, false, true);
            else
                KC_LAUNCH(bf16_t, 2, false, false);
        }
        else
            {
            if (img)
                KC_LAUNCH(bf16_t, 1, false, true);
            else
                KC_LAUNCH(bf16_t, 1, false, false);
        }
    } else {
        if (hist)
            KC_LAUNCH(float, 2, true, false);
        else if (a.causal_t)
            {
            if (img)
                KC_LAUNCH(float, 2, false, true);
            else
                KC_LAUNCH(float, 2, false, false);
        }
        else
            {
            if (img)
                KC_LAUNCH(float, 1, false, true);
            else
                KC_LAUNCH(float, 1, false, false);
        }
    }
#undef KC_LAUNCH
    return hipGetLastError();
}

}  // namespace kdaconv
