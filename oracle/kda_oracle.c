/*
 * Oracle for the gated delta rule with a gate per key dimension (KDA) —
 * TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, plain CPU definition that the GPU library's KDA
 * kernels are checked against. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header or constant with the HIP library, nor with the
 * GDN oracle beside it.
 *
 * What it computes (page "Formulas and code for adapting inference to
 * GDN/KDA linear modules", section 2.1, the recurrent kernel's KDA branch:
 * the gate of a token is a vector over the key dimensions, and the state,
 * laid out with one row per key dimension, has each row scaled by the
 * exponential of that dimension's gate; the rest of the step is the gated
 * delta rule of section 1.1): for every sequence n and head h, from
 * S = S0[n,h] (zeros when none), for each token t in order, with
 * beta_t = beta[t,h]:
 *
 *     S[i][:] <- exp(g[t,h,i]) * S[i][:]   for every key dim i   decay
 *     u       =  k_t^T S                                         what the state holds for k_t
 *     S       <- S + beta_t * k_t (v_t - u)^T                    delta-rule write
 *     o[t]    =  scale * q_t^T S                                 read after the write
 *
 * The decay comes before the memory read, as in the GDN reading (the page's
 * chunkwise form measures the correction against the decayed state, and its
 * recurrent kernel scales the state as soon as it has loaded the gate). The
 * page's pseudocode has no output scale; `scale` is an argument (1 reproduces
 * it). The page normalises q and k inside the call (use_qk_l2norm_in_kernel);
 * here they are used as given and the caller normalises them.
 *
 * Everything is fp64; q, k, v, g, beta arrive as fp32 (bf16 values convert
 * exactly), the initial state as fp64. Layouts: q, k [B,T,H,Dk], v [B,T,H,Dv],
 * g [B,T,H,Dk], beta [B,T,H], states [N,H,Dk,Dv]; packed sequences through
 * cu [N+1] when given (then B = 1 and T is the packed total).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One token on one head's state S (Dk x Dv, row i = key dim i); g holds the
 * token's Dk gate values. */
static void kda_token(double *S, const float *q, const float *k, const float *v, const float *g,
                      double beta, double scale, int Dk, int Dv, double *u, double *o) {
    for (int i = 0; i < Dk; ++i) {
        const double alpha = exp((double)g[i]);
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= alpha;
    }
    for (int j = 0; j < Dv; ++j) u[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
        const double ki = (double)k[i];
        for (int j = 0; j < Dv; ++j) u[j] += ki * S[(size_t)i * Dv + j];
    }
    for (int i = 0; i < Dk; ++i) {
        const double bk = beta * (double)k[i];
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += bk * ((double)v[j] - u[j]);
    }
    for (int j = 0; j < Dv; ++j) o[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
        const double qi = (double)q[i];
        for (int j = 0; j < Dv; ++j) o[j] += qi * S[(size_t)i * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) o[j] *= scale;
}

/* Whole sequences. Returns 0, or -1 on a bad argument / allocation failure. */
int kda_oracle_forward(const float *q, const float *k, const float *v, const float *g,
                       const float *beta, const double *S0, double *o, double *Sfin,
                       const int64_t *cu, int N, int T, int H, int Dk, int Dv, double scale,
                       int nthreads) {
    if (N < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads) reduction(| : bad)
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < H; ++h) {
            double *S = malloc(sizeof(double) * (size_t)Dk * Dv);
            double *u = malloc(sizeof(double) * (size_t)Dv);
            if (!S || !u) {
                free(S);
                free(u);
                bad = 1;
                continue;
            }
            const size_t sbase = ((size_t)n * H + h) * Dk * Dv;
            for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] = S0 ? S0[sbase + e] : 0.0;
            int64_t tok0, len;
            if (cu) {
                tok0 = cu[n];
                len = cu[n + 1] - cu[n];
            } else {
                tok0 = (int64_t)n * T;
                len = T;
            }
            for (int64_t t = tok0; t < tok0 + len; ++t) {
                const size_t th = (size_t)t * H + h;
                kda_token(S, q + th * Dk, k + th * Dk, v + th * Dv, g + th * Dk, (double)beta[th],
                          scale, Dk, Dv, u, o + th * Dv);
            }
            if (Sfin)
                for (size_t e = 0; e < (size_t)Dk * Dv; ++e) Sfin[sbase + e] = S[e];
            free(S);
            free(u);
        }
    return bad ? -1 : 0;
}

/* One decode token per row, on a state pool through a row -> slot map
 * (idx null: row r uses slot r). q, k, g [N,H,Dk]; v [N,H,Dv]; beta [N,H]. */
int kda_oracle_step(const float *q, const float *k, const float *v, const float *g,
                    const float *beta, double *state, const int32_t *idx, double *o, int N, int H,
                    int Dk, int Dv, double scale, int nthreads) {
    if (N < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    int bad = 0;
#pragma omp parallel for collapse(2) num_threads(nthreads) reduction(| : bad)
    for (int r = 0; r < N; ++r)
        for (int h = 0; h < H; ++h) {
            double *u = malloc(sizeof(double) * (size_t)Dv);
            if (!u) {
                bad = 1;
                continue;
            }
            const int64_t slot = idx ? (int64_t)idx[r] : (int64_t)r;
            const size_t rh = (size_t)r * H + h;
            kda_token(state + ((size_t)slot * H + h) * Dk * Dv, q + rh * Dk, k + rh * Dk,
                      v + rh * Dv, g + rh * Dk, (double)beta[rh], scale, Dk, Dv, u, o + rh * Dv);
            free(u);
        }
    return bad ? -1 : 0;
}
