/*
 * kdaconv: modality-aware short convolution + Kimi Delta Attention (KDA)
 * forward pass for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation is the token mixer of the KDA layers of the Chimera hybrid
 * visual diffusion backbone (Chimera: Designing and Chinchilla-Scaling Hybrid
 * Visual Diffusion Transformers; paper.rainbus.top page, "core method" and
 * "method step details" steps (2) and (5); genai-atlas page, "How it works"):
 *
 *   1. a depthwise short convolution injects local context into q, k and v,
 *      run separately per modality: causal 1D over the text tokens, 3D over
 *      the visual tokens on their (t, h, w) latent grid;
 *   2. a per-head gated delta-rule scan over the single raster-ordered stream
 *        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *        o_t = S_t^T q_t
 *      with a channel-wise forget gate alpha_t in (0,1]^dk and a scalar write
 *      strength beta_t.
 *
 * Stream layout: text tokens first, then visual tokens in time-major raster
 * order (w fastest): visual token (t, h, w) sits at stream position
 * n_text + (t * grid_h + h) * grid_w + w.  T = n_text + grid_t*grid_h*grid_w.
 *
 * Tensor layouts (row-major, contiguous, element type given by kda_dtype):
 *   q, k, alpha, q_out, k_out   [B, T, H, dk]
 *   v, v_out, o                 [B, T, H, dv]
 *   beta                        [B, T, H]
 *   w_text[s]                   [H*d_s, k_text]           (s = q, k, v)
 *   w_vis[s]                    [H*d_s, k_vis, k_vis, k_vis]  (t, h, w taps)
 *   initial_state, final_state  float32 [B, H, dk, dv]
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers except the descriptor, which is a host
 *     pointer.  The caller owns all memory.  The library never allocates,
 *     frees or synchronises; work is enqueued on `hip_stream` (a hipStream_t,
 *     NULL = the default stream) and the call returns.  Device faults surface
 *     at the caller's next synchronisation.
 *   - Every argument check runs on the host before any HIP call; a failing
 *     check returns a negative status and enqueues nothing.  Nothing aborts,
 *     exits or throws across the ABI.
 *   - Device pointers must be 16-byte aligned.  Outputs must not overlap any
 *     input (the conv reads neighbours of each token).
 *   - Preconditions that are documented, not checked: 0 < alpha <= 1, all
 *     inputs finite, and within any 8 consecutive tokens of one head the
 *     product of alpha over one key channel stays above 2^-120 (the chunked
 *     scan factorises intra-chunk decays around sub-block midpoints).
 *   - A batch of B = 0 streams enqueues nothing and returns KDA_OK.
 *   - The library is stateless and re-entrant.
 */
#ifndef KDACONV_H
#define KDACONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream structure shared by both entry points. */
typedef struct {
    int32_t n_text;   /* text tokens at the head of the stream (>= 0)            */
    int32_t grid_t;   /* visual latent-patch grid; any extent may be 0 (no video) */
    int32_t grid_h;
    int32_t grid_w;
    int32_t k_text;   /* causal text conv taps; must be 4                         */
    int32_t k_vis;    /* visual conv edge; must be 3 (3x3x3)                     */
    int32_t causal_t; /* 0: symmetric zero padding in t (default); 1: time-causal
                         variant, taps at t-2, t-1, t                            */
} kda_stream_desc;

typedef enum {
    KDA_F32 = 0,      /* fp32 in and out; fp32 arithmetic throughout              */
    KDA_BF16 = 1      /* bf16 in and out; fp32 accumulation                      */
} kda_dtype;

enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null/misaligned/overlapping pointer, bad sizes   */
    KDA_ERR_UNSUPPORTED = -2, /* dk/dv not in {64,128}, k_text != 4, k_vis != 3,
                                 unknown dtype, index space beyond 2^31 tokens    */
    KDA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
    KDA_ERR_HIP = -4          /* a kernel launch reported an error               */
};

/*
 * Modality-aware depthwise short convolution of q, k and v (the conv of the
 * Chimera pages' core method; genai-atlas "How it works": causal 1D depthwise
 * over text tokens, depthwise 3D over visual tokens reshaped to their grid).
 * For each stream s in {q, k, v} and channel c in [0, H*d_s):
 *   text token i < n_text:
 *     out[i, c] = sum_{j=0..3} w_text[s][c, j] * x[i - 3 + j, c]   (x[<0] = 0)
 *   visual token (t, h, w):
 *     out[c] = sum_{a,b,e=0..2} w_vis[s][c, a, b, e] * x(t + a - P, h + b - 1, w + e - 1)
 *     with zero padding outside the grid, P = 1 (symmetric) or 2 (causal_t).
 * The two modalities never read each other.  No bias, no activation.
 * Accumulation is fp32; outputs are rounded to the input dtype (RNE).
 * w_text and w_vis are host arrays of three device pointers each (q, k, v),
 * in the activation dtype.
 */
int kda_conv_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                     kda_dtype dtype, const void *q, const void *k, const void *v,
                     const void *const w_text[3], const void *const w_vis[3],
                     void *q_out, void *k_out, void *v_out, void *hip_stream);

/*
 * The same conv over one segment of a longer time-causal stream (the
 * autoregressive, frame-by-frame use of the time-causal conv that the
 * paper.rainbus.top Chimera page suggests in its limitations section, in the
 * independent-weaknesses and future-directions paragraphs).  A long video is cut
 * along t into segments; each segment is passed as its own stream whose
 * descriptor holds that segment's latent slices (and no text: n_text = 0),
 * with causal_t = 1.  history[s] (device, per q, k, v: [B, n_hist * h * w,
 * H, d_s], the stream dtype, 16-byte aligned) holds the conv INPUTS of the
 * n_hist latent slices just before the segment, oldest first; n_hist = 2
 * makes the segment's outputs equal to the corresponding slices of one pass
 * over the whole stream (n_hist = 0 is the start of a stream, i.e. plain
 * kda_conv_forward).  Together with kda_forward's initial_state/final_state
 * this processes a stream in segments.
 * Errors: KDA_ERR_INVALID_ARG when n_hist is not 0..2, or n_hist > 0 with
 * causal_t != 1, n_text != 0, an empty grid, or a null, misaligned or
 * output-overlapping history pointer; otherwise as kda_conv_forward.
 */
int kda_conv_forward_stream(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                            kda_dtype dtype, const void *q, const void *k, const void *v,
                            const void *const history[3], int n_hist,
                            const void *const w_text[3], const void *const w_vis[3],
                            void *q_out, void *k_out, void *v_out, void *hip_stream);

/* Bytes of device workspace kda_forward needs for this shape: the chunk
 * transforms of every (batch, head, chunk), plus, when the state pass cuts the
 * streams into segments, one record per (batch, head, segment) of fp32
 * 2 dk dv + dk dk values.  Host arithmetic only (no HIP call); the same for
 * every device.  0 on bad or unsupported arguments, including shapes whose
 * per-(batch, head) transforms would reach 4 GiB. */
size_t kda_forward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk,
                                  int dv, kda_dtype dtype);

/*
 * KDA gated delta-rule scan (the state update of the Chimera pages' method step
 * (5); the readout o_t = S_t^T q_t uses the post-update state, no scale).
 * For every batch b and head h, starting from S_0 = initial_state[b, h] (or 0
 * when initial_state is NULL):
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 * o is written in the input dtype; final_state (optional, NULL to skip)
 * receives S_T in fp32.  Supported: dk, dv in {64, 128} in either dtype.  The
 * scan is computed chunkwise (64 tokens per chunk): an intra-chunk kernel forms
 * every chunk's UT/WY transform on matrix cores and writes it to `workspace`;
 * the state pass then cuts each stream's chunks into segments (about
 * 256 / (B H) of them, at most 32), forms each segment's affine state map
 * S -> Phi S + L in parallel, chains the segments' start states in fp32, and
 * replays every segment from its start state, in parallel, writing o.
 * `workspace` (device, >= the size returned by kda_forward_workspace_size) is
 * scratch owned by the caller; its contents are undefined afterwards.
 * initial_state may alias final_state.
 */
int kda_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                kda_dtype dtype, const void *q, const void *k, const void *v,
                const void *alpha, const void *beta, const float *initial_state,
                float *final_state, void *o, void *workspace, size_t workspace_bytes,
                void *hip_stream);

/*
 * kda_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and checks as kda_forward, with the chunk workspace held
 * in the library's own device array of KDA_NOALLOC_SCRATCH_BYTES per device
 * (allocated when the library's code is loaded on a device, kept until the
 * process ends) instead of a caller's buffer.  The call allocates and frees
 * nothing.  Shapes whose workspace (kda_forward_workspace_size) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one device uses that device's one array: calls
 * that overlap in time on one device (different streams, or host threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe.  The first call on a device looks up the array's address
 * (a host-side query, no allocation); a failure there is KDA_ERR_HIP.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int kda_forward_noalloc(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                        kda_dtype dtype, const void *q, const void *k, const void *v,
                        const void *alpha, const void *beta, const float *initial_state,
                        float *final_state, void *o, void *hip_stream);

/*
 * The conv and KDA in one call, with the conv inside the chunk transform: the
 * chunk transform forms the conv outputs q', k', v' of each chunk's rows itself,
 * from the conv inputs q, k, v and the taps (the operations of kda_conv_forward
 * above, summed in fp32 in tap order and rounded to the stream dtype), so they
 * are never written to memory; then the state pass of kda_forward.  This is the
 * conv-into-KDA fusion that follows from the Chimera pages' core method, where
 * the modality-aware short conv feeds every KDA update (genai-atlas "How it
 * works"; paper.rainbus.top 技术新颖性 on the fused conv).  Inputs and outputs
 * as kda_conv_forward (q, k, v, w_text, w_vis) and kda_forward (alpha, beta,
 * initial_state, final_state, o) for a uniform batch; the same errors.
 * Against kda_conv_forward + kda_forward it saves the q', k', v' buffers (3 of
 * the 5 stream-sized activations a step holds) at the price of time: each
 * chunk gathers its 3x3x3 neighbourhoods from the conv inputs through the
 * caches instead of reading q', k', v' once.  o agrees with the two-call path
 * to the rounding of q', k', v' (the two sum the taps in different orders).
 * workspace (device, 16-byte aligned, caller-owned, contents undefined after):
 * at least kda_conv_kda_forward_workspace_size bytes, which is
 * kda_forward_workspace_size rounded up to 256 bytes plus the three streams'
 * taps, 31 per channel in the stream dtype.  KDA_ERR_INVALID_ARG also when a
 * tap array overlaps o, final_state or the workspace, or the workspace
 * overlaps any input or output (the call writes all of the workspace).
 */
size_t kda_conv_kda_forward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk,
                                           int dv, kda_dtype dtype);
int kda_conv_kda_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                         kda_dtype dtype, const void *q, const void *k, const void *v,
                         const void *const w_text[3], const void *const w_vis[3],
                         const void *alpha, const void *beta, const float *initial_state,
                         float *final_state, void *o, void *workspace, size_t workspace_bytes,
                         void *hip_stream);

/*
 * The two stages of kda_forward, callable separately with the same shapes,
 * checks and workspace: kda_forward(...) is exactly kda_forward_chunks(...)
 * followed by kda_forward_scan(...) on one stream.  kda_forward_chunks forms
 * every chunk's UT/WY transform (fully parallel over chunks) and writes it to
 * the workspace; kda_forward_scan runs the segmented state pass (segment
 * maps, chain of start states, replay) and writes o and optionally
 * final_state.  The workspace must not be modified between the two calls.
 */
int kda_forward_chunks(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                       kda_dtype dtype, const void *q, const void *k, const void *v,
                       const void *alpha, const void *beta, void *workspace,
                       size_t workspace_bytes, void *hip_stream);

int kda_forward_scan(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                     kda_dtype dtype, const float *initial_state, float *final_state,
                     void *o, const void *workspace, size_t workspace_bytes,
                     void *hip_stream);

/*
 * Variable-length batches.  n_seq streams (1 <= n_seq <= KDA_MAX_SEQS), each
 * with its own layout descs[i] (T_i >= 1 tokens), packed one after another
 * along the token axis: stream i occupies tokens [P_i, P_i + T_i) with
 * P_i = T_0 + ... + T_{i-1}, so q, k, alpha, q_out, k_out are
 * [sum T_i, H, dk], v, v_out, o are [sum T_i, H, dv] and beta is
 * [sum T_i, H]; initial_state and final_state are float32 [n_seq, H, dk, dv].
 * The streams are independent: each one's conv sees only its own tokens, and
 * each one's scan starts from its own initial state.  The result for stream
 * i equals the uniform entry point called on that stream alone with B = 1.
 * All streams share H, dk, dv and dtype.  (Batches that mix images, videos
 * of different lengths or sizes, and text-only streams are the use.)
 * kda_conv_forward_varlen enqueues one conv launch per stream;
 * kda_forward_varlen enqueues one launch of each KDA kernel for all streams.
 * Errors: KDA_ERR_INVALID_ARG for n_seq < 1 or a NULL descs, and whatever a
 * stream's layout would give with B = 1; KDA_ERR_UNSUPPORTED for
 * n_seq > KDA_MAX_SEQS or a packed axis past the uniform entry points'
 * limits; otherwise as kda_conv_forward / kda_forward.
 */
#define KDA_MAX_SEQS 64
size_t kda_forward_varlen_workspace_size(const kda_stream_desc *descs, int n_seq, int H, int dk,
                                         int dv, kda_dtype dtype);

int kda_forward_varlen(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv,
                       kda_dtype dtype, const void *q, const void *k, const void *v,
                       const void *alpha, const void *beta, const float *initial_state,
                       float *final_state, void *o, void *workspace, size_t workspace_bytes,
                       void *hip_stream);

int kda_conv_forward_varlen(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv,
                            kda_dtype dtype, const void *q, const void *k, const void *v,
                            const void *const w_text[3], const void *const w_vis[3],
                            void *q_out, void *k_out, void *v_out, void *hip_stream);

/*
 * Backward of the KDA scan, for training (the pages train the backbone end to
 * end; they do not describe the mixer's backward, which is the exact gradient
 * of the forward above).  Inputs: the forward's q, k, v (the conv outputs),
 * alpha, beta and initial_state (NULL = 0); the gradient of o, d_o
 * [B, T, H, dv] in the stream dtype; the gradient of the final state,
 * d_final_state (fp32 [B, H, dk, dv], NULL = 0).  Outputs: d_q, d_k
 * [B, T, H, dk], d_v [B, T, H, dv], d_alpha [B, T, H, dk], d_beta [B, T, H]
 * in the stream dtype, and d_initial_state (fp32 [B, H, dk, dv], NULL to
 * skip).  Computed chunk by chunk in fp32: a per-chunk transform, the state
 * at every chunk start, a reverse pass for the state gradients and a
 * per-chunk gradient kernel.  workspace (device, >= the size returned by
 * kda_backward_workspace_size, fp32 records, states and per-workgroup
 * scratch) is owned by the caller; its contents are undefined afterwards.
 * Same shapes and preconditions as kda_forward (dk, dv in {64, 128}, either
 * dtype; the decay of any 8 consecutive tokens of a channel above 2^-120):
 * the decays inside a chunk are split at 16-token block references as in the
 * forward, so a chunk may decay by any amount.  Where alpha is tiny, d_alpha
 * = d(log alpha) / alpha carries the rounding of d(log alpha), a running sum
 * of terms of order one, divided by alpha.
 * Errors: KDA_ERR_INVALID_ARG for a NULL or misaligned required pointer or an
 * output overlapping an input or another output; KDA_ERR_WORKSPACE for a
 * missing or short workspace; otherwise as kda_forward.
 */
/*
 * Backward of kda_conv_forward.  Given the conv inputs q, k, v, the taps and
 * the gradients of the conv outputs (d_q_out, d_k_out, d_v_out, layouts of
 * q_out, k_out, v_out), writes the gradients of the inputs (d_q, d_k, d_v,
 * stream dtype) and of the taps (d_w_text[s] fp32 [H*d_s, 4], d_w_vis[s] fp32
 * [H*d_s, 27], overwritten; summed over the batch).  Each input receives
 * tap * gradient of every output it feeds; each tap the sum of input *
 * output gradient.  Errors as kda_conv_forward, plus KDA_ERR_INVALID_ARG for
 * a NULL, misaligned or overlapping gradient pointer.
 */
int kda_conv_backward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                      const void *q, const void *k, const void *v, const void *const w_text[3],
                      const void *const w_vis[3], const void *d_q_out, const void *d_k_out,
                      const void *d_v_out, void *d_q, void *d_k, void *d_v,
                      float *const d_w_text[3], float *const d_w_vis[3], void *hip_stream);

size_t kda_backward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                                   kda_dtype dtype);

int kda_backward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                 const void *q, const void *k, const void *v, const void *alpha,
                 const void *beta, const float *initial_state, const void *d_o,
                 const float *d_final_state, void *d_q, void *d_k, void *d_v, void *d_alpha,
                 void *d_beta, float *d_initial_state, void *workspace, size_t workspace_bytes,
                 void *hip_stream);

/*
 * Attention core of the MLA layers that fill one of every four token-mixer
 * layers (Chimera pages, paper.rainbus.top, prerequisites section, the
 * Multi-head Latent Attention paragraph): keys and values are decompressed
 * from a latent by plain projections (mla_latent_forward), and every head
 * also sees one key part shared by all heads (K_direct).  Full bidirectional
 * softmax attention within each stream: for stream b, head h, query i,
 *   s_j = scale * (q_nope[b,i,h] . k_nope[b,j,h] + q_dir[b,i,h] . k_dir[b,j])
 *   o[b,i,h] = sum_j softmax_j(s) v[b,j,h]          (j over all T tokens)
 * Layouts (row-major, contiguous): q_nope, k_nope [B, T, H, d_nope];
 * q_dir [B, T, H, d_dir]; k_dir [B, T, d_dir]; v, o [B, T, H, dv].
 * Supported: KDA_BF16 with d_nope = 128, d_dir = 64, dv = 128 (fp32
 * accumulation, o rounded to bf16); anything else is KDA_ERR_UNSUPPORTED.
 * scale must be finite and > 0 (1 / sqrt(d_nope + d_dir) is the usual one).
 * Errors: KDA_ERR_INVALID_ARG for B < 0, T < 1, H < 1, a bad scale, a NULL
 * or misaligned pointer, or o overlapping an input.
 */
int mla_attention_forward(int B, int T, int H, int d_nope, int d_dir, int dv, kda_dtype dtype,
                          const void *q_nope, const void *q_dir, const void *k_nope,
                          const void *k_dir, const void *v, float scale, void *o,
                          void *hip_stream);

/*
 * Latent projections of the MLA layers (Chimera pages, paper.rainbus.top,
 * prerequisites section, the Multi-head Latent Attention paragraph): the
 * hidden state is compressed into a low-dimensional latent, keys and values
 * are decompressed from it, and the key part shared by all heads (K_direct)
 * is projected from the hidden state beside the latent.  With every weight
 * stored as a linear layer's [out_features, in_features] (row-major):
 *   c      = x W_dkv^T     x [rows, d_model], w_dkv [d_c, d_model]  -> c [rows, d_c]
 *   k_dir  = x W_kr^T      w_kr [d_dir, d_model]                    -> k_dir [rows, d_dir]
 *   k_nope = c W_uk^T      w_uk [H * d_nope, d_c]                   -> k_nope [rows, H, d_nope]
 *   v      = c W_uv^T      w_uv [H * dv, d_c]                       -> v [rows, H, dv]
 * rows = B * T tokens; k_nope, k_dir and v are then the inputs of
 * mla_attention_forward.  The latent c is written (bf16) and the
 * decompression reads it back, as the layer's KV cache would hold it.
 * Supported: KDA_BF16 (fp32 accumulation, every output rounded to bf16),
 * d_model a multiple of 32; d_c, d_dir, H * d_nope and H * dv multiples of
 * 64; anything else is KDA_ERR_UNSUPPORTED.  Two launches on hip_stream; the
 * caller owns every buffer.
 * Errors: KDA_ERR_INVALID_ARG for a negative or zero size (rows = 0 is a
 * no-op), a NULL or not 16-byte aligned pointer, or an output overlapping an
 * input or another output.
 */
int mla_latent_forward(int64_t rows, int d_model, int d_c, int d_dir, int H, int d_nope, int dv,
                       kda_dtype dtype, const void *x, const void *w_dkv, const void *w_kr, const void *w_uk,
                       const void *w_uv, void *c, void *k_dir, void *k_nope, void *v, void *hip_stream);

/* Static, human-readable text for a status code. */
const char *kda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDACONV_H */
