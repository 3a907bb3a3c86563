/*
 * A plain C consumer of libkdaconv.so: no Python, no torch, only the HIP
 * runtime's C API for device memory and a stream.  It runs the conv and the
 * KDA scan of one stream read from raw files and writes the results back.
 *
 *   c_abi_demo DIR
 *
 * DIR/meta.txt holds "B H dk dv n_text grid_t grid_h grid_w causal_t dtype"
 * (dtype 0 = fp32, 1 = bf16).  Inputs (raw, row-major, the stream dtype):
 * q k v alpha beta (.bin), w_text_{q,k,v}.bin, w_vis_{q,k,v}.bin.  Outputs:
 * q_out.bin k_out.bin v_out.bin o.bin (stream dtype) and s_final.bin (fp32).
 * Exit status 0 on success; otherwise the failing call and its status text
 * are printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kdaconv.h"

static const char *g_dir;

static int hip_ok(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

/* Read DIR/name (exactly `bytes` bytes) into a new device buffer. */
static void *upload(const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path);
        return NULL;
    }
    void *host = malloc(bytes);
    size_t got = host ? fread(host, 1, bytes, f) : 0;
    fclose(f);
    if (got != bytes) {
        fprintf(stderr, "%s: expected %zu bytes, read %zu\n", path, bytes, got);
        free(host);
        return NULL;
    }
    void *dev = NULL;
    if (!hip_ok(hipMalloc(&dev, bytes), "hipMalloc") ||
        !hip_ok(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device")) {
        free(host);
        return NULL;
    }
    free(host);
    return dev;
}

/* Write `bytes` bytes of device buffer `dev` to DIR/name. */
static int download(const char *name, const void *dev, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", g_dir, name);
    void *host = malloc(bytes);
    if (!host || !hip_ok(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host")) {
        free(host);
        return 0;
    }
    FILE *f = fopen(path, "wb");
    int ok = f && fwrite(host, 1, bytes, f) == bytes;
    if (f) fclose(f);
    free(host);
    if (!ok) fprintf(stderr, "cannot write %s\n", path);
    return ok;
}

static int kda_ok(int status, const char *what) {
    if (status != KDA_OK) {
        fprintf(stderr, "%s: %s (%d)\n", what, kda_status_string(status), status);
        return 0;
    }
    return 1;
}

int main(int argc, char **argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 2;
    }
    g_dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", g_dir);
    FILE *m = fopen(path, "r");
    int B, H, dk, dv, dtype;
    kda_stream_desc d;
    memset(&d, 0, sizeof d);
    if (!m || fscanf(m, "%d %d %d %d %d %d %d %d %d %d", &B, &H, &dk, &dv, &d.n_text, &d.grid_t, &d.grid_h,
                     &d.grid_w, &d.causal_t, &dtype) != 10) {
        fprintf(stderr, "cannot read %s\n", path);
        if (m) fclose(m);
        return 2;
    }
    fclose(m);
    d.k_text = 4;
    d.k_vis = 3;
    const size_t es = dtype == KDA_F32 ? 4 : 2;
    const size_t T = (size_t)d.n_text + (size_t)d.grid_t * d.grid_h * d.grid_w;
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;

    void *q = upload("q.bin", nk * es), *k = upload("k.bin", nk * es), *v = upload("v.bin", nv * es);
    void *alpha = upload("alpha.bin", nk * es), *beta = upload("beta.bin", (size_t)B * T * H * es);
    const void *wt[3] = {upload("w_text_q.bin", (size_t)H * dk * 4 * es), upload("w_text_k.bin", (size_t)H * dk * 4 * es),
                         upload("w_text_v.bin", (size_t)H * dv * 4 * es)};
    const void *wv[3] = {upload("w_vis_q.bin", (size_t)H * dk * 27 * es), upload("w_vis_k.bin", (size_t)H * dk * 27 * es),
                         upload("w_vis_v.bin", (size_t)H * dv * 27 * es)};
    if (!q || !k || !v || !alpha || !beta || !wt[0] || !wt[1] || !wt[2] || !wv[0] || !wv[1] || !wv[2]) return 1;

    void *qc = NULL, *kc = NULL, *vc = NULL, *o = NULL, *ws = NULL;
    float *sT = NULL;
    const size_t ws_bytes = kda_forward_workspace_size(&d, B, H, dk, dv, (kda_dtype)dtype);
    if (ws_bytes == 0) {
        fprintf(stderr, "kda_forward_workspace_size: unsupported shape\n");
        return 1;
    }
    if (!hip_ok(hipMalloc(&qc, nk * es), "hipMalloc") || !hip_ok(hipMalloc(&kc, nk * es), "hipMalloc") ||
        !hip_ok(hipMalloc(&vc, nv * es), "hipMalloc") || !hip_ok(hipMalloc(&o, nv * es), "hipMalloc") ||
        !hip_ok(hipMalloc((void **)&sT, (size_t)B * H * dk * dv * sizeof(float)), "hipMalloc") ||
        !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc"))
        return 1;

    hipStream_t st;
    if (!hip_ok(hipStreamCreate(&st), "hipStreamCreate")) return 1;
    if (!kda_ok(kda_conv_forward(&d, B, H, dk, dv, (kda_dtype)dtype, q, k, v, wt, wv, qc, kc, vc, st),
                "kda_conv_forward"))
        return 1;
    if (!kda_ok(kda_forward(&d, B, H, dk, dv, (kda_dtype)dtype, qc, kc, vc, alpha, beta, NULL, sT, o, ws, ws_bytes,
                            st),
                "kda_forward"))
        return 1;
    if (!hip_ok(hipStreamSynchronize(st), "hipStreamSynchronize")) return 1;

    if (!download("q_out.bin", qc, nk * es) || !download("k_out.bin", kc, nk * es) ||
        !download("v_out.bin", vc, nv * es) || !download("o.bin", o, nv * es) ||
        !download("s_final.bin", sT, (size_t)B * H * dk * dv * sizeof(float)))
        return 1;

    void *all[] = {q, k, v, alpha, beta, (void *)wt[0], (void *)wt[1], (void *)wt[2], (void *)wv[0],
                   (void *)wv[1], (void *)wv[2], qc, kc, vc, o, sT, ws};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) hipFree(all[i]);
    hipStreamDestroy(st);
    printf("ok: B=%d T=%zu H=%d dk=%d dv=%d\n", B, T, H, dk, dv);
    return 0;
}
