// Fused decode step of Simple GLA: one token per row, state updated in place.
//
// Per (row, head) with state slot s (blueprint page, section "B2 lightning-attn
// (Simple GLA)": decay, outer-product update, query; the state comes from the
// request's pool slot and is saved back):
//
//   S[i][j] <- exp(g) * S[i][j] + k_i v_j          o_j = scale * sum_i q_i S[i][j]
//
// This is a streaming read-modify-write of the state with almost no
// arithmetic per byte, so the kernel is built for HBM bandwidth: one workgroup
// per (row, head) state, each thread owning 16-byte column groups of several
// rows, all loads of the state issued before any store, non-temporal
// loads/stores (the state is touched once per step and should not evict other
// data), and the column sums reduced through LDS.
//
// The state is stored in fp32 or in bf16 (the pool's dtype on the same page).
// A bf16 state is loaded, updated and read by the query in fp32, then stored
// rounded to nearest even.
#include "sgla_internal.h"

namespace sgla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte group of a state row: 4 fp32 or 8 bf16 columns, as fp32.
template <typename Ts>
struct StateVec;
template <>
struct StateVec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float *p, float v[4]) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
    static __device__ __forceinline__ void store(float *p, const float v[4]) {
        const f32x4 x = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
    }
};
template <>
struct StateVec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t *p, float v[8]) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(x[j] << 16);
            v[2 * j + 1] = __uint_as_float(x[j] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float v[8]) {
        u32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[j] = (uint32_t)f32_to_bf16(v[2 * j]) | ((uint32_t)f32_to_bf16(v[2 * j + 1]) << 16);
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
    }
};

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

template <typename Tin, int DK, int DV, bool PRO, typename Ts>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, Ts *__restrict__ state, const int32_t *__restrict__ idx,
    Tin *__restrict__ out, int H, float scale, StepPrologue pro) {
    static_assert(!PRO || DK == 128, "the prologue is built for 128-dim heads");
    constexpr int VEC = StateVec<Ts>::N;  // columns per 16-byte group
    constexpr int CG = DV / VEC;          // column groups per state row
    constexpr int RG = 256 / CG;          // row groups
    constexpr int RPT = DK / RG;          // rows per thread
    static_assert(RPT * RG == DK, "row split");
    const int row = blockIdx.x;  // n * H + h
    const int n = row / H;
    const int h = row - n * H;
    const int tid = threadIdx.x;
    const int64_t slot = idx ? (int64_t)idx[n] : (int64_t)n;

    __shared__ float qs[DK], ks[DK], vs[DV];
    __shared__ float red[RG][CG][VEC];
    static_assert(sizeof(qs) + sizeof(ks) + sizeof(vs) + sizeof(red) <= kLdsPerCU / 4,
                  "four workgroups must fit one CU's LDS");
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
    Ts *S = state + (slot * H + h) * (int64_t)DK * DV;
    float reg[RPT][VEC];
#pragma unroll
    for (int m = 0; m < RPT; ++m) StateVec<Ts>::load(S + ((rg + RG * m) * CG + cg) * VEC, reg[m]);
    __syncthreads();
    float vv[VEC], acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        vv[e] = vs[VEC * cg + e];
        acc[e] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int r = rg + RG * m;
        const float kr = ks[r];
        const float qr = qs[r];
        float s[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[e] = fmaf(kr, vv[e], alpha * reg[m][e]);
        StateVec<Ts>::store(S + (r * CG + cg) * VEC, s);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(qr, s[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[rg][cg][e] = acc[e];
    __syncthreads();
    if (tid < DV) {
        const int c = tid / VEC, e = tid % VEC;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += red[r][c][e];
        store_elem(out, (int64_t)row * DV + tid, scale * sum);
    }
}

template <typename Tin, int DK, int DV, bool PRO, typename Ts>
hipError_t launch_k(const void *q, const void *k, const void *v, const float *g, void *state,
                    const int32_t *idx, void *out, int N, int H, float scale,
                    const StepPrologue &pro, hipStream_t st) {
    hipLaunchKernelGGL((recurrent_step_kernel<Tin, DK, DV, PRO, Ts>), dim3((unsigned)(N * H)),
                       dim3(256), 0, st, static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                       static_cast<const Tin *>(v), g, static_cast<Ts *>(state), idx,
                       static_cast<Tin *>(out), H, scale, pro);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV, typename Ts>
hipError_t launch_t(const void *q, const void *k, const void *v, const float *g, void *state,
                    const int32_t *idx, void *out, int N, int H, float scale,
                    const StepPrologue &pro, hipStream_t st) {
    if constexpr (DK == 128)
        if (pro.qw)
            return launch_k<Tin, DK, DV, true, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    return launch_k<Tin, DK, DV, false, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
}

template <typename Tin, typename Ts>
hipError_t launch_dims(const void *q, const void *k, const void *v, const float *g, void *state,
                       const int32_t *idx, void *out, int N, int H, int Dk, int Dv, float scale,
                       const StepPrologue &pro, hipStream_t st) {
    if (Dk == 128 && Dv == 128)
        return launch_t<Tin, 128, 128, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    if (Dk == 128 && Dv == 64)
        return launch_t<Tin, 128, 64, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    if (Dk == 64 && Dv == 128)
        return launch_t<Tin, 64, 128, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
    return launch_t<Tin, 64, 64, Ts>(q, k, v, g, state, idx, out, N, H, scale, pro, st);
}

}  // namespace

hipError_t launch_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                 void *state, bool state_bf16, const int32_t *idx, void *out,
                                 int N, int H, int Dk, int Dv, float scale, bool bf16,
                                 const StepPrologue &pro, hipStream_t st) {
    if (N == 0) return hipSuccess;
    if (bf16) {
        if (state_bf16)
            return launch_dims<uint16_t, uint16_t>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
        return launch_dims<uint16_t, float>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
    }
    if (state_bf16)
        return launch_dims<float, uint16_t>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
    return launch_dims<float, float>(q, k, v, g, state, idx, out, N, H, Dk, Dv, scale, pro, st);
}

}  // namespace sgla
