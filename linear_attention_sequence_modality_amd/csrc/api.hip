// C-ABI entry points: argument validation (host only, before any HIP call)
// and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kdaconv.h"
#include "launch.h"

namespace {

using kdaconv::ConvArgs;
using kdaconv::KdaArgs;

constexpr int64_t kMaxTokens = (int64_t)1 << 31;

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
    if (T * H * d_max * (dtype == KDA_F32 ? 4 : 2) >= ((int64_t)1 << 32)) return KDA_ERR_UNSUPPORTED;
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

// kda_conv_forward and kda_conv_forward_stream: validation, then one launch.
int conv_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                 const void *q, const void *k, const void *v, const void *const history[3], int n_hist,
                 const void *const w_text[3], const void *const w_vis[3], void *q_out, void *k_out,
                 void *v_out, void *hip_stream) {
    int64_t T = 0;
    int rc = check_shape(desc, B, H, dk, dv, dtype, &T);
    if (rc != KDA_OK) return rc;
    if (!w_text || !w_vis) return KDA_ERR_INVALID_ARG;
    const int64_t slice = (int64_t)desc->grid_h * desc->grid_w;
    if (n_hist < 0 || n_hist > 2) return KDA_ERR_INVALID_ARG;
    if (n_hist > 0 && (!history || desc->causal_t != 1 || desc->n_text != 0 || desc->grid_t * slice == 0))
        return KDA_ERR_INVALID_ARG;
    const size_t es = elem_bytes(dtype);
    const int Cs[3] = {H * dk, H * dk, H * dv};
    const void *in[3] = {q, k, v};
    void *out[3] = {q_out, k_out, v_out};
    Range rin[12], rout[3];
    for (int s = 0; s < 3; ++s) {
        if (!in[s] || !out[s] || !w_text[s] || !w_vis[s]) return KDA_ERR_INVALID_ARG;
        if (!aligned16(in[s]) || !aligned16(out[s]) || !aligned16(w_text[s]) || !aligned16(w_vis[s]))
            return KDA_ERR_INVALID_ARG;
        const size_t nbytes = (size_t)B * (size_t)T * (size_t)Cs[s] * es;
        rin[s] = range_of(in[s], nbytes);
        rin[3 + s] = range_of(w_text[s], (size_t)Cs[s] * 4 * es);
        rin[6 + s] = range_of(w_vis[s], (size_t)Cs[s] * 27 * es);
        rin[9 + s] = Range{0, 0};
        if (n_hist > 0) {
            if (!history[s] || !aligned16(history[s])) return KDA_ERR_INVALID_ARG;
            rin[9 + s] = range_of(history[s], (size_t)B * (size_t)n_hist * (size_t)slice * (size_t)Cs[s] * es);
        }
        rout[s] = range_of(out[s], nbytes);
    }
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 12; ++j)
            if (overlaps(rout[i], rin[j])) return KDA_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (overlaps(rout[i], rout[j])) return KDA_ERR_INVALID_ARG;
    }
    if (B == 0) return KDA_OK;

    ConvArgs a;
    for (int s = 0; s < 3; ++s) {
        a.x[s] = in[s];
        a.y[s] = out[s];
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
    int64_t T = 0;
    if (check_shape(desc, B, H, dk, dv, dtype, &T) != KDA_OK) return 0;
    if (dtype == KDA_F32 && (dk != 64 || dv != 64)) return 0;
    const size_t per = kdaconv::kda_chunk_ws_bytes(dk, dv, dtype == KDA_BF16);
    const int64_t nch = (T + kdaconv::kChunk - 1) / kdaconv::kChunk;
    // the state pass addresses one (batch, head)'s chunks with 32-bit offsets
    if ((int64_t)per * nch >= ((int64_t)1 << 32)) return 0;
    return per * (size_t)B * (size_t)H * (size_t)nch;
}

}  // extern "C"

namespace {

// Validation shared by kda_forward, kda_forward_chunks and kda_forward_scan.
// Null input pointers mean "not used by this entry point" (want_* selects
// which groups are required).  Fills *out on success.
int prepare_kda(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                const float *initial_state, const float *final_state, const void *o,
                const void *workspace, size_t workspace_bytes, bool want_inputs, bool want_outputs,
                KdaArgs *out) {
    int64_t T = 0;
    int rc = check_shape(desc, B, H, dk, dv, dtype, &T);
    if (rc != KDA_OK) return rc;
    if (dtype == KDA_F32 && (dk != 64 || dv != 64)) return KDA_ERR_UNSUPPORTED;
    const size_t es = elem_bytes(dtype);
    const size_t BT = (size_t)B * (size_t)T;
    const size_t sbytes = (size_t)B * H * dk * dv * sizeof(float);
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
    const size_t need = kda_forward_workspace_size(desc, B, H, dk, dv, dtype);
    if (need == 0) return KDA_ERR_UNSUPPORTED;
    if (B > 0) {
        if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KDA_ERR_WORKSPACE;
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
    out->B = B;
    out->T = (int)T;
    out->H = H;
    out->dk = dk;
    out->dv = dv;
    out->n_chunks = (int)((T + kdaconv::kChunk - 1) / kdaconv::kChunk);
    out->c0 = 0;
    out->c1 = out->n_chunks;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_forward(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                const float *initial_state, float *final_state, void *o, void *workspace,
                size_t workspace_bytes, void *hip_stream) {
    KdaArgs a;
    int rc = prepare_kda(desc, B, H, dk, dv, dtype, q, k, v, alpha, beta, initial_state, final_state,
                         o, workspace, workspace_bytes, true, true, &a);
    if (rc != KDA_OK || B == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (kdaconv::launch_kda_chunks(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    if (kdaconv::launch_kda_scan(a, dtype == KDA_BF16, st) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

int kda_forward_chunks(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                       const void *q, const void *k, const void *v, const void *alpha,
                       const void *beta, void *workspace, size_t workspace_bytes,
                       void *hip_stream) {
    KdaArgs a;
    int rc = prepare_kda(desc, B, H, dk, dv, dtype, q, k, v, alpha, beta, nullptr, nullptr, nullptr,
                         workspace, workspace_bytes, true, false, &a);
    if (rc != KDA_OK || B == 0) return rc;
    return kdaconv::launch_kda_chunks(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) ==
                   hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

int kda_forward_scan(const kda_stream_desc *desc, int B, int H, int dk, int dv, kda_dtype dtype,
                     const float *initial_state, float *final_state, void *o, const void *workspace,
                     size_t workspace_bytes, void *hip_stream) {
    KdaArgs a;
    int rc = prepare_kda(desc, B, H, dk, dv, dtype, nullptr, nullptr, nullptr, nullptr, nullptr,
                         initial_state, final_state, o, workspace, workspace_bytes, false, true, &a);
    if (rc != KDA_OK || B == 0) return rc;
    return kdaconv::launch_kda_scan(a, dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream)) ==
                   hipSuccess
               ? KDA_OK
               : KDA_ERR_HIP;
}

}  // extern "C"
