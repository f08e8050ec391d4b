/*
 * Oracle for Simple Gated Linear Attention (Simple GLA).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, obviously correct
 * CPU definition that the GPU library is checked against. Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does. It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (page "MiniCPM-SALA — Complete Blueprint", section
 * "B2 lightning-attn (Simple GLA)", steps 1-3 of the per-head recurrence):
 * for every sequence n and head h, independently, starting from the state
 * S = S0[n,h] (zeros when no initial state is given), for each token t of the
 * sequence in order:
 *
 *     S    <- exp(g[t,h]) * S             decay first (scalar x matrix)
 *     S    <- S + k[t,h]^T (x) v[t,h]     rank-1 update, S[i][j] += k_i v_j
 *     o[t] <- scale * (q[t,h] @ S)        query after the update
 *
 * and the state after the last token is the final state. The decay g is the
 * natural-log decay of one token for one head (the page writes alpha =
 * exp(g_gamma[head]) as a fixed per-head constant; here it is an input per
 * token and head, of which the per-head constant is the special case).
 *
 * Everything is fp64. q, k, v, g arrive as fp32 arrays: bf16 values converted
 * to fp32 are exact, so the oracle sees exactly what the GPU receives. The
 * initial state arrives in fp64 so that a final state can be fed back exactly.
 *
 * Layouts (row-major, contiguous):
 *   q, k   [B, T, H, Dk]   (or packed [1, Ttot, H, Dk] when cu_seqlens given)
 *   v      [B, T, H, Dv]
 *   g      [B, T, H]
 *   S0     [N, H, Dk, Dv]  fp64; N = number of sequences; NULL => zeros
 *   o      [B, T, H, Dv]   fp64 out
 *   Sfin   [N, H, Dk, Dv]  fp64 out; NULL => not written
 *   cu     [N + 1] int64 sequence starts in the packed token axis, or NULL
 *          for B rows of T tokens each.
 *
 * Pinned by the CPU tests against: the brute-force causal form when g = 0,
 * the closed-form unrolled final state, split-and-chain, the decay table the
 * blueprint page prints, and the brute-force parallel form with an initial
 * state.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Decay: S <- exp(g) * S, a scalar times the whole Dk x Dv state. */
static void decay(double *S, double g, int Dk, int Dv) {
    const double alpha = exp(g);
    for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] = alpha * S[e];
}

/* Update: S <- S + k^T (x) v, i.e. S[i][j] += k_i * v_j. */
static void update(double *S, const float *k, const float *v, int Dk, int Dv) {
    for (int i = 0; i < Dk; ++i) {
        const double ki = (double)k[i];
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += ki * (double)v[j];
    }
}

/* Query: o[j] = scale * sum_i q_i * S[i][j]. */
static void query(const double *S, const float *q, double scale, int Dk, int Dv, double *o) {
    for (int j = 0; j < Dv; ++j) o[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
        const double qi = (double)q[i];
        for (int j = 0; j < Dv; ++j) o[j] += qi * S[(size_t)i * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) o[j] *= scale;
}

/* One token of the recurrence on one head, in the page's order. */
static void token_step(double *S, const float *q, const float *k, const float *v,
                       double g, double scale, int Dk, int Dv, double *o_out) {
    decay(S, g, Dk, Dv);
    update(S, k, v, Dk, Dv);
    query(S, q, scale, Dk, Dv, o_out);
}

/* Full forward over one or more sequences. Returns 0 on success, -1 on a bad
 * argument, -2 when a state buffer cannot be allocated. */
int sgla_oracle_forward(const float *q, const float *k, const float *v, const float *g,
                        const double *S0, double *o, double *Sfin, const int64_t *cu,
                        int B, int T, int H, int Dk, int Dv, double scale, int nthreads) {
    if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const int N = B;
    const int64_t units = (int64_t)N * H;
    int err = 0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
    for (int64_t u = 0; u < units; ++u) {
        const int n = (int)(u / H);
        const int h = (int)(u % H);
        int64_t tok0, len;
        if (cu) {
            tok0 = cu[n];
            len = cu[n + 1] - cu[n];
        } else {
            tok0 = (int64_t)n * T;
            len = T;
        }
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        if (!S) { err |= 1; continue; }
        const size_t sbase = ((size_t)n * H + h) * (size_t)Dk * Dv;
        for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] = S0 ? S0[sbase + e] : 0.0;
        for (int64_t t = tok0; t < tok0 + len; ++t) {
            const size_t row = (size_t)t * H + h;
            token_step(S, q + row * Dk, k + row * Dk, v + row * Dv, (double)g[row], scale,
                       Dk, Dv, o + row * Dv);
        }
        if (Sfin) memcpy(Sfin + sbase, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
    }
    return err ? -2 : 0;
}

/* One decode step for N rows: row r uses state slot idx[r] (r when idx is
 * NULL), applies the same token body in place on that slot, and writes o[r].
 * q, k [N, H, Dk]; v [N, H, Dv]; g [N, H]; state [slots, H, Dk, Dv] fp64. */
int sgla_oracle_step(const float *q, const float *k, const float *v, const float *g,
                     double *state, const int32_t *idx, double *o, int N, int H, int Dk,
                     int Dv, double scale, int nthreads) {
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const int64_t units = (int64_t)N * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t u = 0; u < units; ++u) {
        const int r = (int)(u / H);
        const int h = (int)(u % H);
        const int64_t slot = idx ? (int64_t)idx[r] : (int64_t)r;
        double *S = state + ((size_t)slot * H + h) * (size_t)Dk * Dv;
        const size_t row = (size_t)r * H + h;
        token_step(S, q + row * Dk, k + row * Dk, v + row * Dv, (double)g[row], scale, Dk,
                   Dv, o + row * Dv);
    }
    return 0;
}
