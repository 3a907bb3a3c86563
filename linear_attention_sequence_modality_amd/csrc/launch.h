// Internal launcher interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kdaconv {

// ---- modality-aware short conv ---------------------------------------------
struct ConvArgs {
    const void *x[3];    // q, k, v inputs   [B, T, C[s]]
    void *y[3];          // q', k', v'       [B, T, C[s]]
    const void *wt[3];   // text taps        [C[s], 4]
    const void *wv[3];   // visual taps      [C[s], 27]
    int C[3];            // channels per stream (H*dk, H*dk, H*dv)
    int B, T, n_text, gt, gh, gw, causal_t;
    // time-causal streaming: the n_hist latent slices just before this
    // segment's first slice, as conv inputs [B, n_hist * gh * gw, C[s]]
    const void *hx[3];
    int n_hist;
};
hipError_t launch_conv(const ConvArgs &a, bool bf16, hipStream_t stream);

// Backward of the conv: dx of the inputs (stream dtype) and fp32 tap gradients.
struct ConvBwdArgs {
    const void *x[3], *dy[3];   // conv inputs, gradients of the conv outputs [B, T, C[s]]
    void *dx[3];                // gradients of the conv inputs
    const void *wt[3], *wv[3];  // taps [C[s], 4] and [C[s], 27]
    float *dwt[3], *dwv[3];     // their gradients, overwritten
    int C[3];
    int B, T, n_text, gt, gh, gw, causal_t;
};
hipError_t launch_conv_backward(const ConvBwdArgs &a, bool bf16, hipStream_t stream);

// ---- chunked KDA -----------------------------------------------------------
constexpr int kChunk = 64;  // tokens per chunk

constexpr int kMaxSeqs = 64;  // sequences of one variable-length batch

// The token axis of q, k, v, alpha, beta and o holds B sequences one after
// another: all of length T (a uniform batch, [B, T, H, d]), or sequence i at
// tokens [tok0[i], tok0[i+1]) (a variable-length batch, [1, sum T_i, H, d]).
// Each sequence is split into chunks of kChunk tokens (its last one ragged);
// the workspace holds chunk g of head h at index h * total chunks + g, where
// sequence i owns chunks [chk0[i], chk0[i+1]).
//
// The state pass cuts each sequence's chunks into segments of consecutive
// chunks (sequence i: seg_len(i) chunks each, the last one shorter), which
// are summarised, chained and replayed in parallel.  The segment records sit
// after the chunk records in the workspace, at byte seg_base: one per
// (head, segment) at index h * total segments + segment, each holding the
// segment's state map (L, Phi) and its start state.
struct KdaArgs {
    const void *q, *k, *v, *alpha, *beta;
    const float *s0;     // [B, H, dk, dv] or null
    float *sT;           // [B, H, dk, dv] or null
    void *o;             // token axis as above, [.., H, dv]
    void *ws;            // chunk workspace
    int B, T, H, dk, dv;
    int n_chunks;        // uniform batch: ceil(T / kChunk)
    int varlen;          // nonzero: the tables below give the sequences
    int tok0[kMaxSeqs + 1], chk0[kMaxSeqs + 1];
    // segments: uniform batch n_seg_u per sequence of seg_len_u chunks; a
    // variable-length batch uses the tables
    int n_seg_u, seg_len_u;
    int seg0[kMaxSeqs + 1], seg_len[kMaxSeqs];
    size_t seg_base;     // byte offset of the segment records in ws
    // The conv inside the chunk transform (launch_kda_chunks_conv, a uniform
    // batch): q, k and v above are the conv INPUTS, and the chunk transform
    // forms q', k', v' itself.  cw + cw_off[s] elements holds stream s's taps
    // tap-major in the stream dtype, [31][C[s]] (visual tap a*9 + b*3 + e, then
    // the 4 text taps), written by launch_conv_taps_tapmajor; n_text, gt, gh, gw
    // give the stream layout and pt the time offset of the visual taps (1:
    // symmetric padding, 2: time-causal).
    const void *cw;
    int cw_off[3];
    int n_text, gt, gh, gw, pt;
};
// First token and first chunk of sequence i (i = B: the totals).
__host__ __device__ inline int seq_tok0(const KdaArgs &a, int i) { return a.varlen ? a.tok0[i] : i * a.T; }
__host__ __device__ inline int seq_chk0(const KdaArgs &a, int i) { return a.varlen ? a.chk0[i] : i * a.n_chunks; }
// First segment of sequence i (i = B: the total), and its segments' length in chunks.
__host__ __device__ inline int seq_seg0(const KdaArgs &a, int i) { return a.varlen ? a.seg0[i] : i * a.n_seg_u; }
__host__ __device__ inline int seq_seg_len(const KdaArgs &a, int i) { return a.varlen ? a.seg_len[i] : a.seg_len_u; }
// Sequence that owns segment g (0 <= g < total segments).
__device__ inline int seq_of_segment(const KdaArgs &a, int g) {
    if (!a.varlen) return g / a.n_seg_u;
    int lo = 0, hi = a.B;   // seg0[lo] <= g < seg0[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.seg0[mid] <= g) lo = mid;
        else hi = mid;
    }
    return lo;
}
// Segment plan: chunks per segment aim at kSegTarget (head, segment) pairs in
// all, at most kMaxSegs segments per sequence (the chain over them is serial).
constexpr int kSegTarget = 256;
constexpr int kMaxSegs = 32;
__host__ __device__ inline int segs_of(int n_chunks, int seg_len) { return (n_chunks + seg_len - 1) / seg_len; }
// Bytes of one segment record: L [dk, dv], Phi [dk, dk], start state [dk, dv], fp32.
__host__ __device__ inline size_t seg_record_bytes(int dk, int dv) { return ((size_t)2 * dk * dv + (size_t)dk * dk) * 4; }
// Sequence that owns chunk g (0 <= g < total chunks).
__device__ inline int seq_of_chunk(const KdaArgs &a, int g) {
    if (!a.varlen) return g / a.n_chunks;
    int lo = 0, hi = a.B;   // chk0[lo] <= g < chk0[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.chk0[mid] <= g) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Workspace bytes for one (batch, head, chunk).
size_t kda_chunk_ws_bytes(int dk, int dv, bool bf16);
// The chunk transform (chunk records into the workspace) and the state pass
// over them (segment summaries, the chain of segment start states, and the
// replay of every segment writing o and the final state).
hipError_t launch_kda_chunks(const KdaArgs &a, bool bf16, hipStream_t stream);
// The chunk transform with the conv in its loader (the conv fields of KdaArgs set).
hipError_t launch_kda_chunks_conv(const KdaArgs &a, bool bf16, hipStream_t stream);
// Taps of the three streams, w_text [C[s], 4] and w_vis [C[s], 27] in the stream
// dtype, into cw tap-major (same dtype): stream s at element off[s], [31][C[s]].
constexpr int kConvTaps = 31;
hipError_t launch_conv_taps_tapmajor(const void *const wt[3], const void *const wv[3], const int Cs[3],
                                     const int off[3], void *cw, bool bf16, hipStream_t stream);
hipError_t launch_kda_scan(const KdaArgs &a, bool bf16, hipStream_t stream);
// Compute units of the current device.
int num_cus();

// ---- KDA backward ----------------------------------------------------------
// Uniform batch [B, T, H, d] as in the forward.  All buffers are caller-owned;
// rec, states, dstates and scratch are parts of one workspace.
struct KdaBwdArgs {
    const void *q, *k, *v, *alpha, *beta, *dO;   // forward inputs and the gradient of o
    const float *s0, *dsT;                       // initial state, gradient of the final state (or null)
    float *sT;                                   // unused by the backward (null)
    void *dq, *dk_out, *dv_out, *dalpha, *dbeta; // gradients, stream dtype
    float *ds0;                                  // gradient of the initial state (or null)
    float *rec, *states, *dstates, *scratch;     // workspace parts (fp32)
    size_t rec_floats, scratch_floats;
    int B, T, H, dk, dv, n_chunks;
};
constexpr int kBwdBlocks = 512;   // workgroups of the two chunk-parallel backward kernels (at most)
size_t kda_bwd_scratch_floats(int dk, int dv);
size_t kda_bwd_rec_floats(int dk, int dv);
hipError_t launch_kda_backward(KdaBwdArgs a, bool bf16, hipStream_t stream);

// ---- MLA attention core ----------------------------------------------------
// q_nope, k_nope [B, T, H, 128]; q_dir [B, T, H, 64]; k_dir [B, T, 64] (shared
// by the heads); v, o [B, T, H, 128]; bf16.
struct MlaArgs {
    const void *q_nope, *q_dir, *k_nope, *k_dir, *v;
    void *o;
    int B, T, H;
    float scale;
};
hipError_t launch_mla_attention(const MlaArgs &a, hipStream_t stream);

// Y = X W^T for two weight/output pairs: X [M, K]; W1 [N1, K] -> Y1 [M, N1];
// W2 [N2, K] -> Y2 [M, N2]; bf16, row-major.  K % 32 == 0, N1 % 64 == 0,
// N2 % 64 == 0, 16-byte aligned rows.
struct MlaProjArgs {
    const void *X, *W1, *W2;
    void *Y1, *Y2;
    int64_t M;
    int K, N1, N2;
};
hipError_t launch_mla_proj(const MlaProjArgs &a, hipStream_t stream);

}  // namespace kdaconv
