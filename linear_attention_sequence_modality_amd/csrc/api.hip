// C-ABI entry points: argument validation (host only, before any HIP call)
// and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kdaconv.h"
#include "launch.h"

namespace {

using kdaconv::ConvArgs;
using kdaconv::KdaArgs;

constexpr int64_t kMaxTokens = (int64_t)1 << 31;
static_assert(kdaconv::kMaxSeqs == KDA_MAX_SEQS, "one limit on the sequences of a batch");

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void *p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(kda_dtype dt) { return dt == KDA_F32 ? 4 : 2; }

// Shared shape validation.  Returns KDA_OK and fills T / sizes, or an error.
int check_shape(const kda_stream_desc *d, int B, int H, int dk, int dv, int dtype, int64_t *T_out) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || H < 1 || d->n_text < 0 || d->grid_t < 0 || d->grid_h < 0 || d->grid_w < 0)
        return KDA_ERR_INVALID_ARG;
    if (d->causal_t != 0 && d->causal_t != 1) return KDA_ERR_INVALID_ARG;
    if (d->k_text != 4 || d->k_vis != 3) return KDA_ERR_UNSUPPORTED;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_UNSUPPORTED;
    const int64_t nv = (int64_t)d->grid_t * d->grid_h * d->grid_w;
    const int64_t T = (int64_t)d->n_text + nv;
    if (T < 1) return KDA_ERR_INVALID_ARG;
    if (T >= kMaxTokens || (int64_t)B * T >= kMaxTokens || H > 4096) return KDA_ERR_UNSUPPORTED;
    // every launch indexes threads and work items with 32-bit integers, and the
    // conv addresses one batch's slice of a stream with 32-bit byte offsets
    const int64_t d_max = dk > dv ? dk : dv;
    if ((int64_t)B * T * H * d_max / 2 >= kMaxTokens) return KDA_ERR_UNSUPPORTED;
    // (plus one chunk: the state pass forms the offsets of a ragged chunk's rows past the end)
    if ((T + kdaconv::kChunk) * H * d_max * (dtype == KDA_F32 ? 4 : 2) >= ((int64_t)1 << 32))
        return KDA_ERR_UNSUPPORTED;
    *T_out = T;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char *kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Pointer checks of a conv call over `tokens` tokens of each stream (plus
// `hist_tokens` history tokens): every pointer set and 16-byte aligned, and no
// output overlapping an input, a weight, a history buffer or another output.
int conv_check_pointers(int64_t tokens, int64_t hist_tokens, const int Cs[3], size_t es, const void *const in[3],
                        const void *const history[3], const void *const w_text[3], const void *const w_vis[3],
                        void *const out[3]) {
    if (!w_text || !w_vis) return KDA_ERR_INVALID_ARG;
    Range rin[12], rout[3];
    for (int s = 0; s < 3; ++s) {
        if (!in[s] || !out[s] || !w_text[s] || !w_vis[s]) return KDA_ERR_INVALID_ARG;
        if (!aligned16(in[s]) || !aligned16(out[s]) || !aligned16(w_text[s]) || !aligned16(w_vis[s]))
            return KDA_ERR_INVALID_ARG;
        const size_t nbytes = (size_t)tokens * (size_t)Cs[s] * es;
        rin[s] = range_of(in[s], nbytes);
        rin[3 + s] = range_of(w_text[s], (size_t)Cs[s] * 4 * es);
        rin[6 + s] = range_of(w_vis[s], (size_t)Cs[s] * 27 * es);
        rin[9 + s] = Range{0, 0};
        if (hist_tokens > 0) {
            if (!history[s] || !aligned16(history[s])) return KDA_ERR_INVALID_ARG;
            rin[9 + s] = range_of(history[s], (size_t)hist_tokens * (size_t)Cs[s] * es);
        }
        rout[s] = range_of(out[s], nbytes);
    }
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 12; ++j)
            if (overlaps(rout[i], rin[j])) return KDA_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlaps(rout[i], rout[j])) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

// One conv launch over B streams of desc's layout (T tokens each) whose first
// token is token `tok` of the arrays (a validated call).
int conv_launch(const kda_stream_desc *desc, int B, int64_t T, int64_t tok, const int Cs[3], kda_dtype dtype,
                const void *const in[3], const void *const history[3], int n_hist,
                const void *const w_text[3], const void *const w_vis[3], void *const out[3],
                void *hip_stream) {
    const size_t es = elem_bytes(dtype);
    ConvArgs a;
    for (int s = 0; s < 3; ++s) {
        const size_t off = (size_t)tok * (size_t)Cs[s] * es;
        a.x[s] = static_cast<const char *>(in[s]) + off;
        a.y[s] = static_cast<char *>(out[s]) + off;
        a.wt[s] = w_text[s];
        a.wv[s] = w_vis[s];
        a.C[s] = Cs[s];
        a.hx[s] = n_hist > 0 ? history[s] : nullptr;
    }
    a.B = B;
    a.T = (int)T;
    a.n_text = desc->n_text;
    a.gt = desc->grid_t;
    a.gh = desc->grid_h;
    a.gw = desc->grid_w;
    if ((int64_t)desc->grid_t * desc->grid_h * desc->grid_w == 0) a.gt = a.gh = a.gw = 0;
    a.causal_t = desc->causal_t;
    a.n_hist = n_hist;
    hipError_t e = kdaconv::launch_conv(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// kda_conv_forward and kda_conv_forward_stream: validation, then one launch.
int conv_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                 const void *q, const void *k, const void *v, const void *const history[3], int n_hist,
                 const void *const w_text[3], const void *const w_vis[3], void *q_out, void *k_out,
                 void *v_out, void *hip_stream) {
    int64_t T = 0;
    int rc = check_shape(desc, B, H, dk, dv, dtype, &T);
    if (rc != KDA_OK) return rc;
    const int64_t slice = (int64_t)desc->grid_h * desc->grid_w;
    if (n_hist < 0 || n_hist > 2) return KDA_ERR_INVALID_ARG;
    if (n_hist > 0 && (!history || desc->causal_t != 1 || desc->n_text != 0 || desc->grid_t * slice == 0))
        return KDA_ERR_INVALID_ARG;
    const int Cs[3] = {H * dk, H * dk, H * dv};
    const void *in[3] = {q, k, v};
    void *out[3] = {q_out, k_out, v_out};
    rc = conv_check_pointers((int64_t)B * T, (int64_t)B * n_hist * slice, Cs, elem_bytes(dtype), in, history,
                             w_text, w_vis, out);
    if (rc != KDA_OK || B == 0) return rc;
    return conv_launch(desc, B, T, 0, Cs, dtype, in, history, n_hist, w_text, w_vis, out, hip_stream);
}

// The sequences of one KDA call: B streams of one layout (a uniform batch) or
// up to kMaxSeqs streams with their own layouts packed along the token axis
// (a variable-length batch).
struct Seqs {
    int n = 0;               // sequences
    int T = 0;               // uniform batch: tokens per sequence
    bool varlen = false;
    int64_t tokens = 0;      // over all sequences
    int64_t chunks = 0;      // over all sequences
    int64_t max_chunks = 0;  // of the longest sequence
    int tok0[kdaconv::kMaxSeqs + 1] = {}, chk0[kdaconv::kMaxSeqs + 1] = {};
};

int64_t chunks_of(int64_t T) { return (T + kdaconv::kChunk - 1) / kdaconv::kChunk; }

int uniform_seqs(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype, Seqs *sq) {
    int64_t T = 0;
    int rc = check_shape(desc, B, H, dk, dv, dtype, &T);
    if (rc != KDA_OK) return rc;
    sq->n = B;
    sq->T = (int)T;
    sq->tokens = (int64_t)B * T;
    sq->max_chunks = chunks_of(T);
    sq->chunks = (int64_t)B * sq->max_chunks;
    return KDA_OK;
}

int varlen_seqs(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv, kda_dtype dtype, Seqs *sq) {
    if (!descs || n_seq < 1) return KDA_ERR_INVALID_ARG;
    if (n_seq > kdaconv::kMaxSeqs) return KDA_ERR_UNSUPPORTED;
    int64_t tok = 0, chk = 0;
    for (int i = 0; i < n_seq; ++i) {
        int64_t T = 0;
        int rc = check_shape(&descs[i], 1, H, dk, dv, dtype, &T);
        if (rc != KDA_OK) return rc;
        sq->tok0[i] = (int)tok;
        sq->chk0[i] = (int)chk;
        tok += T;
        chk += chunks_of(T);
        if (chunks_of(T) > sq->max_chunks) sq->max_chunks = chunks_of(T);
        // the packed token axis obeys the limits of one batch of tok tokens
        const int64_t d_max = dk > dv ? dk : dv;
        if (tok >= kMaxTokens || tok * H * d_max / 2 >= kMaxTokens) return KDA_ERR_UNSUPPORTED;
    }
    sq->tok0[n_seq] = (int)tok;
    sq->chk0[n_seq] = (int)chk;
    sq->n = n_seq;
    sq->varlen = true;
    sq->tokens = tok;
    sq->chunks = chk;
    return KDA_OK;
}

// Segments of the state pass: each sequence's chunks are cut into runs of
// about total chunk-heads / kSegTarget chunks (at most kMaxSegs runs per
// sequence), so that the replay has about one workgroup per compute unit.
struct SegPlan {
    int n_seg_u = 1, seg_len_u = 1;   // uniform batch
    int seg0[kdaconv::kMaxSeqs + 1] = {}, seg_len[kdaconv::kMaxSeqs] = {};
    int64_t total = 0;                // segments over all sequences
};

void plan_segment(int64_t n_chunks, int64_t target_len, int *n_seg, int *seg_len) {
    int64_t p = (n_chunks + target_len - 1) / target_len;
    if (p > kdaconv::kMaxSegs) p = kdaconv::kMaxSegs;
    if (p < 1) p = 1;
    const int64_t len = (n_chunks + p - 1) / p;
    *seg_len = (int)len;
    *n_seg = kdaconv::segs_of((int)n_chunks, (int)len);
}

SegPlan plan_segments(const Seqs &sq, int H) {
    SegPlan sp;
    const int64_t work = sq.chunks * H;
    const int64_t target_len = work > kdaconv::kSegTarget ? (work + kdaconv::kSegTarget - 1) / kdaconv::kSegTarget : 1;
    if (!sq.varlen) {
        plan_segment(sq.max_chunks, target_len, &sp.n_seg_u, &sp.seg_len_u);
        sp.total = (int64_t)sq.n * sp.n_seg_u;
        return sp;
    }
    int64_t g = 0;
    for (int i = 0; i < sq.n; ++i) {
        int n_seg = 1;
        plan_segment(sq.chk0[i + 1] - sq.chk0[i], target_len, &n_seg, &sp.seg_len[i]);
        sp.seg0[i] = (int)g;
        g += n_seg;
    }
    sp.seg0[sq.n] = (int)g;
    sp.total = g;
    return sp;
}

// Byte offset of the segment records (after the chunk records), and the
// workspace bytes of a call, or 0 when the configuration is unsupported.
size_t chunk_records_bytes(const Seqs &sq, int H, int dk, int dv, kda_dtype dtype) {
    const size_t per = kdaconv::kda_chunk_ws_bytes(dk, dv, dtype == KDA_BF16);
    return (per * (size_t)H * (size_t)sq.chunks + 255) / 256 * 256;
}

size_t workspace_bytes_of(const Seqs &sq, int H, int dk, int dv, kda_dtype dtype) {
    const size_t per = kdaconv::kda_chunk_ws_bytes(dk, dv, dtype == KDA_BF16);
    // the state pass addresses one (sequence, head)'s chunks with 32-bit offsets
    if ((int64_t)per * sq.max_chunks >= ((int64_t)1 << 32)) return 0;
    const SegPlan sp = plan_segments(sq, H);
    size_t bytes = chunk_records_bytes(sq, H, dk, dv, dtype);
    if (sp.total > sq.n) bytes += (size_t)sp.total * H * kdaconv::seg_record_bytes(dk, dv);
    return bytes;
}

}  // namespace

extern "C" {

int kda_conv_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                     const void *q, const void *k, const void *v, const void *const w_text[3],
                     const void *const w_vis[3], void *q_out, void *k_out, void *v_out,
                     void *hip_stream) {
    return conv_forward(desc, B, H, dk, dv, dtype, q, k, v, nullptr, 0, w_text, w_vis, q_out, k_out, v_out,
                        hip_stream);
}

int kda_conv_forward_stream(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                            const void *q, const void *k, const void *v, const void *const history[3],
                            int n_hist, const void *const w_text[3], const void *const w_vis[3], void *q_out,
                            void *k_out, void *v_out, void *hip_stream) {
    return conv_forward(desc, B, H, dk, dv, dtype, q, k, v, history, n_hist, w_text, w_vis, q_out, k_out, v_out,
                        hip_stream);
}

size_t kda_forward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                                  kda_dtype dtype) {
    Seqs sq;
    if (uniform_seqs(desc, B, H, dk, dv, dtype, &sq) != KDA_OK) return 0;
    return workspace_bytes_of(sq, H, dk, dv, dtype);
}

size_t kda_forward_varlen_workspace_size(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv,
                                         kda_dtype dtype) {
    Seqs sq;
    if (varlen_seqs(descs, n_seq, H, dk, dv, dtype, &sq) != KDA_OK) return 0;
    return workspace_bytes_of(sq, H, dk, dv, dtype);
}

}  // extern "C"

namespace {

// Validation shared by kda_forward, kda_forward_chunks, kda_forward_scan and
// kda_forward_varlen, for the sequences sq (checked already).  Null input
// pointers mean "not used by this entry point" (want_* selects which groups
// are required).  Fills *out on success.
int prepare_kda(const Seqs &sq, int H, int dk, int dv, kda_dtype dtype, const void *q, const void *k,
                const void *v, const void *alpha, const void *beta, const float *initial_state,
                const float *final_state, const void *o, const void *workspace, size_t workspace_bytes,
                bool want_inputs, bool want_outputs, KdaArgs *out, bool own_scratch = false) {
    const size_t es = elem_bytes(dtype);
    const size_t BT = (size_t)sq.tokens;
    const size_t sbytes = (size_t)sq.n * H * dk * dv * sizeof(float);
    Range rin[6] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}, {0, 0}, {0, 0}};
    if (want_inputs) {
        const void *ins[5] = {q, k, v, alpha, beta};
        for (int i = 0; i < 5; ++i)
            if (!ins[i] || !aligned16(ins[i])) return KDA_ERR_INVALID_ARG;
        rin[0] = range_of(q, BT * H * dk * es);
        rin[1] = range_of(k, BT * H * dk * es);
        rin[2] = range_of(v, BT * H * dv * es);
        rin[3] = range_of(alpha, BT * H * dk * es);
        rin[4] = range_of(beta, BT * H * es);
    }
    Range ro{0, 0}, rs{0, 0};
    if (want_outputs) {
        if (!o || !aligned16(o)) return KDA_ERR_INVALID_ARG;
        if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
            return KDA_ERR_INVALID_ARG;
        if (initial_state) rin[5] = range_of(initial_state, sbytes);
        ro = range_of(o, BT * H * dv * es);
        if (final_state) rs = range_of(final_state, sbytes);
        for (int i = 0; i < 6; ++i)
            if (overlaps(ro, rin[i])) return KDA_ERR_INVALID_ARG;
        for (int i = 0; i < 5; ++i)
            if (overlaps(rs, rin[i])) return KDA_ERR_INVALID_ARG;
        if (final_state && initial_state && final_state != initial_state && overlaps(rs, rin[5]))
            return KDA_ERR_INVALID_ARG;
        if (overlaps(rs, ro)) return KDA_ERR_INVALID_ARG;
    }
    if (sq.n > 0) {
        const size_t need = workspace_bytes_of(sq, H, dk, dv, dtype);
        if (need == 0) return KDA_ERR_UNSUPPORTED;
        if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    }
    if (sq.n > 0 && !own_scratch) {
        const size_t need = workspace_bytes_of(sq, H, dk, dv, dtype);
        if (!workspace || !aligned16(workspace)) return KDA_ERR_WORKSPACE;
        const Range rw = range_of(workspace, need);
        for (int i = 0; i < 6; ++i)
            if (overlaps(rw, rin[i])) return KDA_ERR_INVALID_ARG;
        if (overlaps(rw, ro) || overlaps(rw, rs)) return KDA_ERR_INVALID_ARG;
    }
    out->q = q;
    out->k = k;
    out->v = v;
    out->alpha = alpha;
    out->beta = beta;
    out->s0 = initial_state;
    out->sT = const_cast<float *>(final_state);
    out->o = const_cast<void *>(o);
    out->ws = const_cast<void *>(workspace);
    out->B = sq.n;
    out->T = sq.T;
    out->H = H;
    out->dk = dk;
    out->dv = dv;
    out->n_chunks = sq.varlen ? 0 : (int)sq.max_chunks;
    out->varlen = sq.varlen ? 1 : 0;
    for (int i = 0; i <= kdaconv::kMaxSeqs; ++i) {
        out->tok0[i] = sq.tok0[i];
        out->chk0[i] = sq.chk0[i];
    }
    const SegPlan sp = plan_segments(sq, H);
    out->n_seg_u = sp.n_seg_u;
    out->seg_len_u = sp.seg_len_u;
    for (int i = 0; i <= kdaconv::kMaxSeqs; ++i) out->seg0[i] = sp.seg0[i];
    for (int i = 0; i < kdaconv::kMaxSeqs; ++i) out->seg_len[i] = sp.seg_len[i];
    out->seg_base = chunk_records_bytes(sq, H, dk, dv, dtype);
    // no conv inside the chunk transform unless kda_conv_kda_forward sets it up
    out->cw = nullptr;
    for (int s = 0; s < 3; ++s) out->cw_off[s] = 0;
    out->n_text = out->gt = out->gh = out->gw = 0;
    out->pt = 1;
    return KDA_OK;
}

// kda_forward and kda_forward_varlen: both kernels on one stream.
int forward(const Seqs &sq, int H, int dk, int dv, kda_dtype dtype, const void *q, const void *k,
            const void *v, const void *alpha, const void *beta, const float *initial_state, float *final_state,
            void *o, void *workspace, size_t workspace_bytes, void *hip_stream) {
    KdaArgs a;
    int rc = prepare_kda(sq, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state, o, workspace,
                         workspace_bytes, true, true, &a);
    if (rc != KDA_OK || sq.n == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (kdaconv::launch_kda_chunks(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    if (kdaconv::launch_kda_scan(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                const float *initial_state, float *final_state, void *o, void *workspace,
                size_t workspace_bytes, void *hip_stream) {
    Seqs sq;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc != KDA_OK) return rc;
    return forward(sq, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state, o, workspace,
                   workspace_bytes, hip_stream);
}

// The fused entry point's workspace: kda_forward's, then the three streams' taps
// tap-major (31 per channel, the stream dtype), 256-byte aligned.
static size_t conv_taps_bytes(int H, int dk, int dv, kda_dtype dtype) {
    return ((size_t)kdaconv::kConvTaps * (size_t)(2 * H * dk + H * dv) * elem_bytes(dtype) + 255) / 256 * 256;
}

size_t kda_conv_kda_forward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk, int dv,
                                           kda_dtype dtype) {
    Seqs sq;
    if (uniform_seqs(desc, B, H, dk, dv, dtype, &sq) != KDA_OK) return 0;
    const size_t ws = workspace_bytes_of(sq, H, dk, dv, dtype);
    return ws ? (ws + 255) / 256 * 256 + conv_taps_bytes(H, dk, dv, dtype) : 0;
}

int kda_conv_kda_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                         const void *q, const void *k, const void *v, const void *const w_text[3],
                         const void *const w_vis[3], const void *alpha, const void *beta,
                         const float *initial_state, float *final_state, void *o, void *workspace,
                         size_t workspace_bytes, void *hip_stream) {
    Seqs sq;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc != KDA_OK) return rc;
    // the taps: set, aligned, and not overlapping the outputs (checked with the rest below)
    if (!w_text || !w_vis) return KDA_ERR_INVALID_ARG;
    const int Cs[3] = {H * dk, H * dk, H * dv};
    const size_t es = elem_bytes(dtype);
    for (int s = 0; s < 3; ++s)
        if (!w_text[s] || !w_vis[s] || !aligned16(w_text[s]) || !aligned16(w_vis[s])) return KDA_ERR_INVALID_ARG;
    const size_t need = kda_conv_kda_forward_workspace_size(desc, B, H, dk, dv, dtype);
    if (B > 0 && need == 0) return KDA_ERR_UNSUPPORTED;
    if (B > 0 && workspace_bytes < need) return KDA_ERR_WORKSPACE;
    KdaArgs a;
    rc = prepare_kda(sq, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state, o, workspace,
                     workspace_bytes, true, true, &a);
    if (rc != KDA_OK) return rc;
    if (B == 0) return KDA_OK;
    const size_t kda_ws = (workspace_bytes_of(sq, H, dk, dv, dtype) + 255) / 256 * 256;
    const Range ro = range_of(o, (size_t)sq.tokens * H * dv * es);
    const Range rs = final_state ? range_of(final_state, (size_t)B * H * dk * dv * sizeof(float)) : Range{0, 0};
    // the whole fused workspace (chunk records, then the tap-major taps) clear of the taps,
    // the other inputs and the outputs: the call writes all of it
    const Range rall = range_of(workspace, need);
    for (int s = 0; s < 3; ++s) {
        const Range rw[2] = {range_of(w_text[s], (size_t)Cs[s] * 4 * es), range_of(w_vis[s], (size_t)Cs[s] * 27 * es)};
        for (const Range &r : rw)
            if (overlaps(r, ro) || overlaps(r, rs) || overlaps(r, rall)) return KDA_ERR_INVALID_ARG;
    }
    const Range rin[5] = {range_of(q, (size_t)sq.tokens * Cs[0] * es), range_of(k, (size_t)sq.tokens * Cs[1] * es),
                          range_of(v, (size_t)sq.tokens * Cs[2] * es), range_of(alpha, (size_t)sq.tokens * Cs[0] * es),
                          range_of(beta, (size_t)sq.tokens * H * es)};
    for (const Range &r : rin)
        if (overlaps(rall, r)) return KDA_ERR_INVALID_ARG;
    if (overlaps(rall, ro) || overlaps(rall, rs)) return KDA_ERR_INVALID_ARG;
    const int off[3] = {0, Cs[0] * kdaconv::kConvTaps, 2 * Cs[0] * kdaconv::kConvTaps};
    void *cw = static_cast<char *>(workspace) + kda_ws;
    a.cw = cw;
    for (int s = 0; s < 3; ++s) a.cw_off[s] = off[s];
    a.n_text = desc->n_text;
    a.gt = desc->grid_t;
    a.gh = desc->grid_h;
    a.gw = desc->grid_w;
    if ((int64_t)desc->grid_t * desc->grid_h * desc->grid_w == 0) a.gt = a.gh = a.gw = 0;
    a.pt = desc->causal_t ? 2 : 1;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (kdaconv::launch_conv_taps_tapmajor(w_text, w_vis, Cs, off, cw, dtype == KDA_BF16, st) != hipSuccess)
        return KDA_ERR_HIP;
    if (kdaconv::launch_kda_chunks_conv(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    if (kdaconv::launch_kda_scan(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

int kda_forward_varlen(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv, kda_dtype dtype,
                       const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                       const float *initial_state, float *final_state, void *o, void *workspace,
                       size_t workspace_bytes, void *hip_stream) {
    Seqs sq;
    int rc = varlen_seqs(descs, n_seq, H, dk, dv, dtype, &sq);
    if (rc != KDA_OK) return rc;
    return forward(sq, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state, o, workspace,
                   workspace_bytes, hip_stream);
}

}  // extern "C"

namespace {

// ---- the allocation-free forward --------------------------------------------
// kda_forward_noalloc keeps its chunk workspace in this file-scope device
// array instead of a caller's buffer.  Each device that loads the library
// holds its own copy until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = (size_t)64 << 20;   // KDA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "one stated scratch size");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device.
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_forward_noalloc(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                        const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                        const float *initial_state, float *final_state, void *o, void *hip_stream) {
    Seqs sq;
    KdaArgs a;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc == KDA_OK)
        rc = prepare_kda(sq, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state, o, nullptr,
                         kScratchBytes, true, true, &a, true);
    if (rc != KDA_OK || B == 0) return rc;
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != KDA_OK) return rc;
    a.ws = ws;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (kdaconv::launch_kda_chunks(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    if (kdaconv::launch_kda_scan(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

int kda_forward_chunks(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                       const void *q, const void *k, const void *v, const void *alpha,
                       const void *beta, void *workspace, size_t workspace_bytes,
                       void *hip_stream) {
    Seqs sq;
    KdaArgs a;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc == KDA_OK)
        rc = prepare_kda(sq, H, dk, dv, dtype, q, k, v, alpha, beta, nullptr, nullptr, nullptr, workspace,
                         workspace_bytes, true, false, &a);
    if (rc != KDA_OK || B == 0) return rc;
    return kdaconv::launch_kda_chunks(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) ==
                   hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

int kda_forward_scan(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                     const float *initial_state, float *final_state, void *o, const void *workspace,
                     size_t workspace_bytes, void *hip_stream) {
    Seqs sq;
    KdaArgs a;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc == KDA_OK)
        rc = prepare_kda(sq, H, dk, dv, dtype, nullptr, nullptr, nullptr, nullptr, nullptr, initial_state,
                         final_state, o, workspace, workspace_bytes, false, true, &a);
    if (rc != KDA_OK || B == 0) return rc;
    return kdaconv::launch_kda_scan(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) ==
                   hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

int kda_conv_forward_varlen(const kda_stream_desc *descs, int n_seq, int H, int dk, int dv, kda_dtype dtype,
                            const void *q, const void *k, const void *v, const void *const w_text[3],
                            const void *const w_vis[3], void *q_out, void *k_out, void *v_out,
                            void *hip_stream) {
    Seqs sq;
    int rc = varlen_seqs(descs, n_seq, H, dk, dv, dtype, &sq);
    if (rc != KDA_OK) return rc;
    const int Cs[3] = {H * dk, H * dk, H * dv};
    const void *in[3] = {q, k, v};
    void *out[3] = {q_out, k_out, v_out};
    rc = conv_check_pointers(sq.tokens, 0, Cs, elem_bytes(dtype), in, nullptr, w_text, w_vis, out);
    if (rc != KDA_OK) return rc;
    // one launch per sequence, in order on the caller's stream
    for (int i = 0; i < n_seq; ++i) {
        rc = conv_launch(&descs[i], 1, sq.tok0[i + 1] - sq.tok0[i], sq.tok0[i], Cs, dtype, in, nullptr, 0, w_text,
                         w_vis, out, hip_stream);
        if (rc != KDA_OK) return rc;
    }
    return KDA_OK;
}

int mla_attention_forward(int B, int T, int H, int d_nope, int d_dir, int dv, kda_dtype dtype, const void *q_nope,
                          const void *q_dir, const void *k_nope, const void *k_dir, const void *v, float scale,
                          void *o, void *hip_stream) {
    if (B < 0 || T < 1 || H < 1) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (dtype != KDA_BF16 || d_nope != 128 || d_dir != 64 || dv != 128) return KDA_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !(scale < INFINITY)) return KDA_ERR_INVALID_ARG;
    // token and block indices stay in 32 bits, and so do the byte offsets inside one
    // batch's keys and values (the kernel reads them through 32-bit buffer ranges)
    if ((int64_t)B * T * H * 128 >= kMaxTokens * 2 || (int64_t)B * H * ((T + 127) / 128) >= kMaxTokens ||
        (int64_t)T * H * 128 * 2 >= kMaxTokens * 2)
        return KDA_ERR_UNSUPPORTED;
    const void *ins[5] = {q_nope, q_dir, k_nope, k_dir, v};
    const size_t es = 2, BT = (size_t)B * (size_t)T;
    const size_t nbytes[5] = {BT * H * d_nope * es, BT * H * d_dir * es, BT * H * d_nope * es, BT * d_dir * es,
                              BT * H * dv * es};
    if (!o || !aligned16(o)) return KDA_ERR_INVALID_ARG;
    const Range ro = range_of(o, BT * H * dv * es);
    for (int i = 0; i < 5; ++i) {
        if (!ins[i] || !aligned16(ins[i])) return KDA_ERR_INVALID_ARG;
        if (overlaps(ro, range_of(ins[i], nbytes[i]))) return KDA_ERR_INVALID_ARG;
    }
    if (B == 0) return KDA_OK;
    kdaconv::MlaArgs a;
    a.q_nope = q_nope;
    a.q_dir = q_dir;
    a.k_nope = k_nope;
    a.k_dir = k_dir;
    a.v = v;
    a.o = o;
    a.B = B;
    a.T = T;
    a.H = H;
    a.scale = scale;
    return kdaconv::launch_mla_attention(a, static_cast<hipStream_t>(hip_stream)) == hipSuccess ? KDA_OK
                                                                                               : KDA_ERR_HIP;
}

int mla_latent_forward(int64_t rows, int d_model, int d_c, int d_dir, int H, int d_nope, int dv,
                       kda_dtype dtype, const void *x, const void *w_dkv, const void *w_kr, const void *w_uk,
                       const void *w_uv, void *c, void *k_dir, void *k_nope, void *v, void *hip_stream) {
    if (rows < 0 || d_model < 1 || d_c < 1 || d_dir < 1 || H < 1 || d_nope < 1 || dv < 1)
        return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    // the projection kernel's tiling: contraction in steps of 32, output columns in tiles of 64
    if (d_model % 32 || d_c % 64 || d_dir % 64 || ((int64_t)H * d_nope) % 64 || ((int64_t)H * dv) % 64)
        return KDA_ERR_UNSUPPORTED;
    const int64_t nk = (int64_t)H * d_nope, nv = (int64_t)H * dv;
    if (nk + nv > (1 << 20) || d_model > (1 << 20) || d_c > (1 << 20) ||
        (rows + 255) / 256 * ((nk + nv) / 64) >= kMaxTokens)
        return KDA_ERR_UNSUPPORTED;
    const size_t es = 2, R = (size_t)rows;
    const void *ins[5] = {x, w_dkv, w_kr, w_uk, w_uv};
    const size_t in_bytes[5] = {R * d_model * es, (size_t)d_c * d_model * es, (size_t)d_dir * d_model * es,
                                (size_t)nk * d_c * es, (size_t)nv * d_c * es};
    void *outs[4] = {c, k_dir, k_nope, v};
    const size_t out_bytes[4] = {R * d_c * es, R * d_dir * es, R * nk * es, R * nv * es};
    for (int i = 0; i < 5; ++i)
        if (!ins[i] || !aligned16(ins[i])) return KDA_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i) {
        if (!outs[i] || !aligned16(outs[i])) return KDA_ERR_INVALID_ARG;
        const Range ro = range_of(outs[i], out_bytes[i]);
        for (int j = 0; j < 5; ++j)
            if (overlaps(ro, range_of(ins[j], in_bytes[j]))) return KDA_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlaps(ro, range_of(outs[j], out_bytes[j]))) return KDA_ERR_INVALID_ARG;
    }
    if (rows == 0) return KDA_OK;
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    kdaconv::MlaProjArgs down;
    down.X = x;
    down.W1 = w_dkv;
    down.W2 = w_kr;
    down.Y1 = c;
    down.Y2 = k_dir;
    down.M = rows;
    down.K = d_model;
    down.N1 = d_c;
    down.N2 = d_dir;
    if (kdaconv::launch_mla_proj(down, st) != hipSuccess) return KDA_ERR_HIP;
    kdaconv::MlaProjArgs up;
    up.X = c;
    up.W1 = w_uk;
    up.W2 = w_uv;
    up.Y1 = k_nope;
    up.Y2 = v;
    up.M = rows;
    up.K = d_c;
    up.N1 = (int)nk;
    up.N2 = (int)nv;
    return kdaconv::launch_mla_proj(up, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---- backward ----------------------------------------------------------------

}  // extern "C"

namespace {

struct BwdLayout {
    size_t rec, states, scratch_blocks, total_floats;
    int n_chunks;
};

BwdLayout bwd_layout(int64_t T, int B, int H, int dk, int dv) {
    BwdLayout L;
    L.n_chunks = (int)chunks_of(T);
    const size_t items = (size_t)B * H * L.n_chunks;
    L.rec = items * kdaconv::kda_bwd_rec_floats(dk, dv);
    L.states = items * (size_t)dk * dv;
    // per-workgroup scratch of the two chunk-parallel kernels (the ordered passes work in LDS)
    L.scratch_blocks = items < (size_t)kdaconv::kBwdBlocks ? items : (size_t)kdaconv::kBwdBlocks;
    L.total_floats = L.rec + 2 * L.states + L.scratch_blocks * kdaconv::kda_bwd_scratch_floats(dk, dv);
    return L;
}

}  // namespace

extern "C" {

size_t kda_backward_workspace_size(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype) {
    Seqs sq;
    if (uniform_seqs(desc, B, H, dk, dv, dtype, &sq) != KDA_OK) return 0;
    return bwd_layout(sq.T, B, H, dk, dv).total_floats * sizeof(float);
}

int kda_backward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype, const void *q,
                 const void *k, const void *v, const void *alpha, const void *beta, const float *initial_state,
                 const void *d_o, const float *d_final_state, void *d_q, void *d_k, void *d_v, void *d_alpha,
                 void *d_beta, float *d_initial_state, void *workspace, size_t workspace_bytes, void *hip_stream) {
    Seqs sq;
    int rc = uniform_seqs(desc, B, H, dk, dv, dtype, &sq);
    if (rc != KDA_OK) return rc;
    const size_t es = elem_bytes(dtype), BT = (size_t)sq.tokens;
    const size_t sbytes = (size_t)B * H * dk * dv * sizeof(float);
    const void *ins[8] = {q, k, v, alpha, beta, d_o, initial_state, d_final_state};
    const size_t inb[8] = {BT * H * dk * es, BT * H * dk * es, BT * H * dv * es, BT * H * dk * es, BT * H * es,
                           BT * H * dv * es, sbytes, sbytes};
    void *outs[6] = {d_q, d_k, d_v, d_alpha, d_beta, d_initial_state};
    const size_t outb[6] = {BT * H * dk * es, BT * H * dk * es, BT * H * dv * es, BT * H * dk * es, BT * H * es,
                            sbytes};
    Range rin[8], rout[6];
    for (int i = 0; i < 8; ++i) {
        const bool optional = i >= 6;
        if ((!ins[i] && !optional) || (ins[i] && !aligned16(ins[i]))) return KDA_ERR_INVALID_ARG;
        rin[i] = ins[i] ? range_of(ins[i], inb[i]) : Range{0, 0};
    }
    for (int i = 0; i < 6; ++i) {
        const bool optional = i == 5;
        if ((!outs[i] && !optional) || (outs[i] && !aligned16(outs[i]))) return KDA_ERR_INVALID_ARG;
        rout[i] = outs[i] ? range_of(outs[i], outb[i]) : Range{0, 0};
        for (int j = 0; j < 8; ++j)
            if (overlaps(rout[i], rin[j])) return KDA_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlaps(rout[i], rout[j])) return KDA_ERR_INVALID_ARG;
    }
    if (B == 0) return KDA_OK;
    const BwdLayout L = bwd_layout(sq.T, B, H, dk, dv);
    const size_t need = L.total_floats * sizeof(float);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KDA_ERR_WORKSPACE;
    const Range rw = range_of(workspace, need);
    for (int i = 0; i < 8; ++i)
        if (overlaps(rw, rin[i])) return KDA_ERR_INVALID_ARG;
    for (int i = 0; i < 6; ++i)
        if (overlaps(rw, rout[i])) return KDA_ERR_INVALID_ARG;
    kdaconv::KdaBwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.dO = d_o;
    a.s0 = initial_state;
    a.dsT = d_final_state;
    a.sT = nullptr;
    a.dq = d_q;
    a.dk_out = d_k;
    a.dv_out = d_v;
    a.dalpha = d_alpha;
    a.dbeta = d_beta;
    a.ds0 = d_initial_state;
    float *w = static_cast<float *>(workspace);
    a.rec = w;
    a.states = w + L.rec;
    a.dstates = a.states + L.states;
    a.scratch = a.dstates + L.states;
    a.rec_floats = kdaconv::kda_bwd_rec_floats(dk, dv);
    a.scratch_floats = kdaconv::kda_bwd_scratch_floats(dk, dv);
    a.B = B;
    a.T = sq.T;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.n_chunks = L.n_chunks;
    return kdaconv::launch_kda_backward(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

int kda_conv_backward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype, const void *q,
                      const void *k, const void *v, const void *const w_text[3], const void *const w_vis[3],
                      const void *d_q_out, const void *d_k_out, const void *d_v_out, void *d_q, void *d_k, void *d_v,
                      float *const d_w_text[3], float *const d_w_vis[3], void *hip_stream) {
    int64_t T = 0;
    int rc = check_shape(desc, B, H, dk, dv, dtype, &T);
    if (rc != KDA_OK) return rc;
    if (!w_text || !w_vis || !d_w_text || !d_w_vis) return KDA_ERR_INVALID_ARG;
    const size_t es = elem_bytes(dtype);
    const int Cs[3] = {H * dk, H * dk, H * dv};
    const void *x[3] = {q, k, v}, *dy[3] = {d_q_out, d_k_out, d_v_out};
    void *dx[3] = {d_q, d_k, d_v};
    Range rin[12], rout[9];
    for (int s = 0; s < 3; ++s) {
        const size_t nbytes = (size_t)B * (size_t)T * (size_t)Cs[s] * es;
        const void *req[5] = {x[s], dy[s], w_text[s], w_vis[s], dx[s]};
        for (int i = 0; i < 5; ++i)
            if (!req[i] || !aligned16(req[i])) return KDA_ERR_INVALID_ARG;
        if (!d_w_text[s] || !d_w_vis[s] || !aligned16(d_w_text[s]) || !aligned16(d_w_vis[s])) return KDA_ERR_INVALID_ARG;
        rin[s] = range_of(x[s], nbytes);
        rin[3 + s] = range_of(dy[s], nbytes);
        rin[6 + s] = range_of(w_text[s], (size_t)Cs[s] * 4 * es);
        rin[9 + s] = range_of(w_vis[s], (size_t)Cs[s] * 27 * es);
        rout[s] = range_of(dx[s], nbytes);
        rout[3 + s] = range_of(d_w_text[s], (size_t)Cs[s] * 4 * sizeof(float));
        rout[6 + s] = range_of(d_w_vis[s], (size_t)Cs[s] * 27 * sizeof(float));
    }
    for (int i = 0; i < 9; ++i) {
        for (int j = 0; j < 12; ++j)
            if (overlaps(rout[i], rin[j])) return KDA_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlaps(rout[i], rout[j])) return KDA_ERR_INVALID_ARG;
    }
    if (B == 0) return KDA_OK;
    kdaconv::ConvBwdArgs a;
    for (int s = 0; s < 3; ++s) {
        a.x[s] = x[s];
        a.dy[s] = dy[s];
        a.dx[s] = dx[s];
        a.wt[s] = w_text[s];
        a.wv[s] = w_vis[s];
        a.dwt[s] = d_w_text[s];
        a.dwv[s] = d_w_vis[s];
        a.C[s] = Cs[s];
    }
    a.B = B;
    a.T = (int)T;
    a.n_text = desc->n_text;
    a.gt = desc->grid_t;
    a.gh = desc->grid_h;
    a.gw = desc->grid_w;
    if ((int64_t)desc->grid_t * desc->grid_h * desc->grid_w == 0) a.gt = a.gh = a.gw = 0;
    a.causal_t = desc->causal_t;
    return kdaconv::launch_conv_backward(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

}  // extern "C"
