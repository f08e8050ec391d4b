// Fused decode step of the gated delta rule (GDN, and KDA with one gate per
// key dim): one token per row, state updated in place through the row ->
// slot map.
//
// Per (row, head) (page "Formulas and code for adapting inference to GDN/KDA
// linear modules", section 1.1 "Recursive Formulas"; the decay is applied
// before the memory read, as in the page's chunkwise form):
//
//   S <- exp(g) S ;  u = k^T S ;  S <- S + beta k (v - u)^T ;  o = scale q^T S
//
// With per-dim gates (section 2.1, the recurrent kernel's KDA branch) g is a
// vector over the key dims and row i of S is scaled by exp(g[i]).
//
// Like the Simple GLA step this is one read and one write of the fp32 state
// with little arithmetic, built for HBM bandwidth: one workgroup per (row,
// head), each thread owning float4 column groups of several rows, all state
// loads issued before any store. The memory read u needs every row of a
// column, so it takes a reduction through LDS between the load and the
// update; the output takes a second one.
#include "sgla_internal.h"

namespace sgla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename Tin, int DK, int DV, bool KDA>
__global__ __launch_bounds__(256) void gdn_step_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    const int32_t *__restrict__ idx, Tin *__restrict__ out, int H, float scale) {
    constexpr int CG = DV / 4;    // float4 column groups per state row
    constexpr int RG = 256 / CG;  // row groups
    constexpr int RPT = DK / RG;  // rows per thread
    static_assert(RPT * RG == DK, "row split");
    const int row = blockIdx.x;  // n * H + h
    const int n = row / H;
    const int h = row - n * H;
    const int tid = threadIdx.x;
    const int64_t slot = idx ? (int64_t)idx[n] : (int64_t)n;

    __shared__ float qs[DK], ks[DK], vs[DV], es[KDA ? DK : 1];
    __shared__ f32x4 red_u[RG][CG], red_o[RG][CG];
    static_assert(sizeof(qs) + sizeof(ks) + sizeof(vs) + sizeof(es) + sizeof(red_u) + sizeof(red_o) <=
                      kLdsPerCU / 4,
                  "four workgroups must fit one CU's LDS");
    if (tid < DK) {
        qs[tid] = load_elem(q, (int64_t)row * DK + tid);
        ks[tid] = load_elem(k, (int64_t)row * DK + tid);
        if (KDA) es[tid] = __expf(g[(int64_t)row * DK + tid]);
    }
    if (tid < DV) vs[tid] = load_elem(v, (int64_t)row * DV + tid);
    const float alpha = KDA ? 1.f : __expf(g[row]);
    const float b = beta[row];

    const int cg = tid % CG;
    const int rg = tid / CG;
    f32x4 *S = reinterpret_cast<f32x4 *>(state + (slot * H + h) * (int64_t)DK * DV);
    f32x4 reg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) reg[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * CG + cg]);
    __syncthreads();
    // Decay, and this thread's part of u = k^T S over its rows.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        reg[m] *= KDA ? es[rg + RG * m] : alpha;
        const float kr = ks[rg + RG * m];
        acc.x = fmaf(kr, reg[m].x, acc.x);
        acc.y = fmaf(kr, reg[m].y, acc.y);
        acc.z = fmaf(kr, reg[m].z, acc.z);
        acc.w = fmaf(kr, reg[m].w, acc.w);
    }
    red_u[rg][cg] = acc;
    __syncthreads();
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RG; ++r) u += red_u[r][cg];
    // The write beta k (v - u)^T, the store, and this thread's part of q^T S.
    const f32x4 vv = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
    const f32x4 dv = (vv - u) * b;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        const float kr = ks[r];
        const float qr = qs[r];
        f32x4 s;
        s.x = fmaf(kr, dv.x, reg[m].x);
        s.y = fmaf(kr, dv.y, reg[m].y);
        s.z = fmaf(kr, dv.z, reg[m].z);
        s.w = fmaf(kr, dv.w, reg[m].w);
        __builtin_nontemporal_store(s, &S[r * CG + cg]);
        acc.x = fmaf(qr, s.x, acc.x);
        acc.y = fmaf(qr, s.y, acc.y);
        acc.z = fmaf(qr, s.z, acc.z);
        acc.w = fmaf(qr, s.w, acc.w);
    }
    red_o[rg][cg] = acc;
    __syncthreads();
    if (tid < DV) {
        const int c = tid / 4, e = tid % 4;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += red_o[r][c][e];
        store_elem(out, (int64_t)row * DV + tid, scale * sum);
    }
}

template <typename Tin, bool KDA>
hipError_t launch_dims(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, float *state, const int32_t *idx, void *out, int N,
                       int H, int Dk, int Dv, float scale, hipStream_t st) {
    const dim3 grid((unsigned)(N * H)), block(256);
    const Tin *qp = static_cast<const Tin *>(q), *kp = static_cast<const Tin *>(k);
    const Tin *vp = static_cast<const Tin *>(v);
    Tin *op = static_cast<Tin *>(out);
    if (Dk == 128 && Dv == 128)
        hipLaunchKernelGGL((gdn_step_kernel<Tin, 128, 128, KDA>), grid, block, 0, st, qp, kp, vp, g, beta, state, idx, op, H, scale);
    else if (Dk == 128 && Dv == 64)
        hipLaunchKernelGGL((gdn_step_kernel<Tin, 128, 64, KDA>), grid, block, 0, st, qp, kp, vp, g, beta, state, idx, op, H, scale);
    else if (Dk == 64 && Dv == 128)
        hipLaunchKernelGGL((gdn_step_kernel<Tin, 64, 128, KDA>), grid, block, 0, st, qp, kp, vp, g, beta, state, idx, op, H, scale);
    else
        hipLaunchKernelGGL((gdn_step_kernel<Tin, 64, 64, KDA>), grid, block, 0, st, qp, kp, vp, g, beta, state, idx, op, H, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, const int32_t *idx, void *out, int N,
                           int H, int Dk, int Dv, float scale, bool bf16, bool per_dim_gate,
                           hipStream_t st) {
    if (N == 0) return hipSuccess;
    if (per_dim_gate) {
        if (bf16) return launch_dims<uint16_t, true>(q, k, v, g, beta, state, idx, out, N, H, Dk, Dv, scale, st);
        return launch_dims<float, true>(q, k, v, g, beta, state, idx, out, N, H, Dk, Dv, scale, st);
    }
    if (bf16) return launch_dims<uint16_t, false>(q, k, v, g, beta, state, idx, out, N, H, Dk, Dv, scale, st);
    return launch_dims<float, false>(q, k, v, g, beta, state, idx, out, N, H, Dk, Dv, scale, st);
}

}  // namespace sgla
