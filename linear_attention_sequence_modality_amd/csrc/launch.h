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

// ---- chunked KDA -----------------------------------------------------------
constexpr int kChunk = 64;  // tokens per chunk

struct KdaArgs {
    const void *q, *k, *v, *alpha, *beta;
    const float *s0;     // [B, H, dk, dv] or null
    float *sT;           // [B, H, dk, dv] or null
    void *o;             // [B, T, H, dv]
    void *ws;            // chunk workspace
    int B, T, H, dk, dv;
    int n_chunks;        // ceil(T / kChunk)
    int c0, c1;          // chunks [c0, c1) of every (batch, head) processed by one launch
};

// Workspace bytes for one (batch, head, chunk).
size_t kda_chunk_ws_bytes(int dk, int dv, bool bf16);
// Kernel 1 (chunk transform -> workspace) and kernel 2 (ordered state pass).
hipError_t launch_kda_chunks(const KdaArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_kda_scan(const KdaArgs &a, bool bf16, hipStream_t stream);
// Compute units of the current device.
int num_cus();

}  // namespace kdaconv
