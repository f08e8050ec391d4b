// Fused decode step of Simple GLA: one token per row, state updated in place.
//
// Per (row, head) with state slot s (blueprint page, section "B2 lightning-attn
// (Simple GLA)": decay, outer-product update, query; the state comes from the
// request's pool slot and is saved back):
//
//   S[i][j] <- exp(g) * S[i][j] + k_i v_j          o_j = scale * sum_i q_i S[i][j]
//
// This is a streaming read-modify-write of the fp32 state with almost no
// arithmetic per byte, so the kernel is built for HBM bandwidth: one workgroup
// per (row, head) state, each thread owning float4 column groups of several
// rows, all loads of the state issued before any store, non-temporal
// loads/stores (the state is touched once per step and should not evict other
// data), and the column sums reduced through LDS.
#include "sgla_internal.h"

namespace sgla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// The q/k prologue for one head's 128-vector (q in wave 0, k in wave 1): lane
// l holds dims l and l + 64, the pair that RoPE turns together. RMSNorm over
// the 128 dims, weight, bf16; then the turn by pos * theta^(-2l/128), bf16.
// Writes the two results to dst[l] and dst[l + 64].
__device__ __forceinline__ void step_prologue(float a, float b, const float *__restrict__ w,
                                              int64_t pos, const StepPrologue &pro, int l,
                                              float *dst) {
    const float ss = wave_sum(a * a + b * b);
    const float rs = rsqrtf(ss * (1.f / 128) + pro.eps);
    a = round_bf16(a * rs * w[l]);
    b = round_bf16(b * rs * w[l + 64]);
    const float t = rope_base_turns(pos, rope_turns_per_pos(l, 128, pro.theta));
    const float c = cos_turns(t), sn = sin_turns(t);
    dst[l] = round_bf16(fmaf(a, c, -b * sn));
    dst[l + 64] = round_bf16(fmaf(b, c, a * sn));
}

template <typename Tin, int DK, int DV, bool PRO>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, float *__restrict__ state, const int32_t *__restrict__ idx,
    Tin *__restrict__ out, int H, float scale, StepPrologue pro) {
    static_assert(!PRO || DK == 128, "the prologue is built for 128-dim heads");
    constexpr int CG = DV / 4;     // float4 column groups per state row
    constexpr int RG = 256 / CG;   // row groups
    constexpr int RPT = DK / RG;   // rows per thread
    static_assert(RPT * RG == DK, "row split");
    const int row = blockIdx.x;  // n * H + h
    const int n = row / H;
    const int h = row - n * H;
    const int tid = threadIdx.x;
    const int64_t slot = idx ? (int64_t)idx[n] : (int64_t)n;

    __shared__ float qs[DK], ks[DK], vs[DV];
    __shared__ f32x4 red[RG][CG];
    if (PRO) {
        if (tid < 128) {
            const int l = tid & 63;
            const bool isq = tid < 64;
            const Tin *src = (isq ? q : k) + (int64_t)row * DK;
            step_prologue(load_elem(src, l), load_elem(src, l + 64), isq ? pro.qw : pro.kw,
                          (int64_t)pro.pos[n], pro, l, isq ? qs : ks);
        }
    } else if (tid < DK) {
        qs[tid] = load_elem(q, (int64_t)row * DK + tid);
        ks[tid] = load_elem(k, (int64_t)row * DK + tid);
    }
    if (tid < DV) vs[tid] = load_elem(v, (int64_t)row * DV + tid);
    const float alpha = __expf(g[row]);

    const int cg = tid % CG;
    const int rg = tid / CG;
    f32x4 *S = reinterpret_cast<f32x4 *>(state + (slot * H + h) * (int64_t)DK * DV);
    f32x4 reg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) reg[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * CG + cg]);
    __syncthreads();
    const f32x4 vv = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        const float kr = ks[r];
        const float qr = qs[r];
        f32x4 s;
        s.x = fmaf(kr, vv.x, alpha * reg[m].x);
        s.y = fmaf(kr, vv.y, alpha * reg[m].y);
        s.z = fmaf(kr, vv.z, alpha * reg[m].z);
        s.w = fmaf(kr, vv.w, alpha * reg[m].w);
        __builtin_nontemporal_store(s, &S[r * CG + cg]);
        acc.x = fmaf(qr, s.x, acc.x);
        acc.y = fmaf(qr, s.y, acc.y);
        acc.z = fmaf(qr, s.z, acc.z);
        acc.w = fmaf(qr, s.w, acc.w);
    }
    red[rg][cg] = acc;
    __syncthreads();
    if (tid < DV) {
        const int c = tid / 4, e = tid % 4;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += red[r][c][e];
        store_elem(out, (int64_t)row * DV + tid, scale * sum);
    }
}

template <typename Tin, int DK, int DV, bool PRO>
hipError_t launch_k(const void *q, const void *k, const void *v, const float *g, float *state,
                    const int32_t *idx, void *out, int N, int H, float scale,
                    const StepPrologue &pro, hipStream_t st) {
    hipLaunchKernelGGL((recurrent_step_kernel<Tin, DK, DV, PRO>), dim3((unsigned)(N * H)),
                       dim3(256), 0, st, static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                       static_cast<const Tin *>(v), g, state, idx, static_cast<Tin *>(out), H,
                       scale, pro);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV>
hipError_t launch_t(const void *q, const void *k, const void *v, const float *g, float *state,
                    const int32_t *idx, void *out, int N, int H, float scale,
                    const StepPrologue &pro, hipStream_t st) {
    if constexpr (DK == 128)
        if (pro.qw) return launch_k<Tin, DK, DV, true>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    return launch_k<Tin, DK, DV, false>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
}

template <typename Tin>
hipError_t launch_dims(const void *q, const void *k, const void *v, const float *g, float *state,
                       const int32_t *idx, void *out, int N, int H, int Dk, int Dv, float scale,
                       const StepPrologue &pro, hipStream_t st) {
    if (Dk == 128 && Dv == 128)
        return launch_t<Tin, 128, 128>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    if (Dk == 128 && Dv == 64)
        return launch_t<Tin, 128, 64>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    if (Dk == 64 && Dv == 128)
        return launch_t<Tin, 64, 128>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    return launch_t<Tin, 64, 64>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
}

}  // namespace

hipError_t launch_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                 float *state, const int32_t *idx, void *out, int N, int H,
                                 int Dk, int Dv, float scale, bool bf16, const StepPrologue &pro,
                                 hipStream_t st) {
    if (N == 0) return hipSuccess;
    if (bf16) return launch_dims<uint16_t>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
    return launch_dims<float>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
}

}  // namespace sgla
