/*
 * CPU oracle for the modality-aware short convolution + Kimi Delta Attention
 * (KDA) forward pass.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no code with the HIP path.
 *
 * Everything is plain sequential fp64 arithmetic written straight from the
 * definitions (Chimera: Designing and Chinchilla-Scaling Hybrid Visual
 * Diffusion Transformers, paper.rainbus.top page, "core method" and
 * "method step details" steps (2) and (5); genai-atlas page, "How it works").
 * OpenMP only distributes independent (batch, head) scans and independent
 * channels; it never reorders the arithmetic of one output.
 *
 * Readings of points the pages leave open:
 *  - readout o_t = S_t^T q_t with the post-update state, no 1/sqrt(dk) scale;
 *  - q, k and v each go through their own depthwise conv, alpha and beta are
 *    not convolved, there is no bias and no activation after the conv;
 *  - text conv: causal, taps w[0..K-1] applied to x[i-K+1 .. i] (last tap on
 *    the current token), zero left padding, text tokens only;
 *  - visual conv: taps w[a][b][e] applied to x[t+a-P][h+b-1][w+e-1] with zero
 *    padding outside the grid, P = 1 (symmetric, default) or P = 2
 *    (time-causal variant); it never reads text tokens;
 *  - alpha scales the rows (key channels) of S; S_0 = 0 unless given.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); returns the count now in effect. */
int oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * Depthwise modality-aware short convolution of one projected stream.
 *   x, y    : [B, T, channels], T = n_text + grid_t*grid_h*grid_w
 *   w_text  : [channels, k_text]
 *   w_vis   : [channels, k_vis, k_vis, k_vis]  (t, h, w tap order)
 * Text token i (i < n_text):
 *   y[i, c] = sum_j w_text[c, j] * x[i - (k_text - 1) + j, c], terms with
 *   negative index dropped.
 * Visual token (t, h, w) at stream position n_text + (t*grid_h + h)*grid_w + w:
 *   y[c] = sum_{a,b,e} w_vis[c, a, b, e] * x(t + a - pt, h + b - ph, w + e - pw)
 *   with ph = pw = (k_vis - 1) / 2, pt = ph (symmetric) or k_vis - 1 (causal),
 *   terms outside the grid dropped.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_short_conv(int B, int n_text, int grid_t, int grid_h, int grid_w,
                      int channels, int k_text, int k_vis, int causal_t,
                      const double *x, const double *w_text, const double *w_vis,
                      double *y)
{
    if (B < 0 || n_text < 0 || grid_t < 0 || grid_h < 0 || grid_w < 0 ||
        channels <= 0 || k_text <= 0 || k_vis <= 0 || (k_vis % 2) == 0)
        return -1;
    const long T = (long)n_text + (long)grid_t * grid_h * grid_w;
    const int ph = (k_vis - 1) / 2, pw = ph, pt = causal_t ? k_vis - 1 : ph;
    const long nv = (long)grid_t * grid_h * grid_w;

    for (int b = 0; b < B; ++b) {
        const double *xb = x + (size_t)b * T * channels;
        double *yb = y + (size_t)b * T * channels;
#pragma omp parallel for schedule(static)
        for (long i = 0; i < n_text; ++i) {
            for (int c = 0; c < channels; ++c) {
                double acc = 0.0;
                for (int j = 0; j < k_text; ++j) {
                    long src = i - (k_text - 1) + j;
                    if (src < 0)
                        continue;
                    acc += w_text[(size_t)c * k_text + j] * xb[(size_t)src * channels + c];
                }
                yb[(size_t)i * channels + c] = acc;
            }
        }
#pragma omp parallel for schedule(static)
        for (long p = 0; p < nv; ++p) {
            const int t = (int)(p / ((long)grid_h * grid_w));
            const int h = (int)((p / grid_w) % grid_h);
            const int w = (int)(p % grid_w);
            for (int c = 0; c < channels; ++c) {
                const double *wc = w_vis + (size_t)c * k_vis * k_vis * k_vis;
                double acc = 0.0;
                for (int a = 0; a < k_vis; ++a) {
                    const int ts = t + a - pt;
                    if (ts < 0 || ts >= grid_t)
                        continue;
                    for (int bb = 0; bb < k_vis; ++bb) {
                        const int hs = h + bb - ph;
                        if (hs < 0 || hs >= grid_h)
                            continue;
                        for (int e = 0; e < k_vis; ++e) {
                            const int ws = w + e - pw;
                            if (ws < 0 || ws >= grid_w)
                                continue;
                            const long src = n_text + ((long)ts * grid_h + hs) * grid_w + ws;
                            acc += wc[(a * k_vis + bb) * k_vis + e] *
                                   xb[(size_t)src * channels + c];
                        }
                    }
                }
                yb[(size_t)(n_text + p) * channels + c] = acc;
            }
        }
    }
    return 0;
}

/*
 * KDA gated delta rule, plain sequential recurrence per (batch, head).
 *   q, k, alpha : [B, T, H, dk]      v, o : [B, T, H, dv]      beta : [B, T, H]
 *   S0, ST      : [B, H, dk, dv] (either may be NULL: S0 = 0 / not returned)
 * For t = 0 .. T-1 (state update of method step (5), written out as a delta
 * rule):
 *   S'     = Diag(alpha_t) S            (row i of S scaled by alpha_t[i])
 *   u      = beta_t * (v_t - S'^T k_t)
 *   S      = S' + k_t u^T                = (I - beta k k^T) Diag(alpha) S + beta k v^T
 *   o_t    = S^T q_t
 * Returns 0, -1 on a bad argument, -2 on allocation failure.
 */
int oracle_kda_recurrence(int B, int T, int H, int dk, int dv,
                          const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta,
                          const double *S0, double *o, double *ST)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !u) {
            free(S);
            free(u);
            fail |= 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + (size_t)bh * dk * dv, sizeof(double) * (size_t)dk * dv);
        else
            memset(S, 0, sizeof(double) * (size_t)dk * dv);

        for (int t = 0; t < T; ++t) {
            const size_t row = (size_t)b * T + t;
            const double *qt = q + (row * H + h) * dk;
            const double *kt = k + (row * H + h) * dk;
            const double *at = alpha + (row * H + h) * dk;
            const double *vt = v + (row * H + h) * dv;
            const double bt = beta[row * H + h];
            double *ot = o + (row * H + h) * dv;

            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] *= at[i];
            for (int j = 0; j < dv; ++j) {
                double r = 0.0;
                for (int i = 0; i < dk; ++i)
                    r += S[(size_t)i * dv + j] * kt[i];
                u[j] = bt * (vt[j] - r);
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] += kt[i] * u[j];
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i)
                    acc += S[(size_t)i * dv + j] * qt[i];
                ot[j] = acc;
            }
        }
        if (ST)
            memcpy(ST + (size_t)bh * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(u);
    }
    return fail ? -2 : 0;
}
