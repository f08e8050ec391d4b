// Output epilogue of a lightning layer: per token, RMSNorm over the
// concatenated heads and a sigmoid gate (page "MiniCPM-SALA — Complete
// Blueprint", section "B2 lightning-attn (Simple GLA)", step "Output Norm +
// Gate + Projection", without the projection):
//
//   y = o / sqrt(mean(o^2) + eps) * w        (w: one weight per column)
//   out = y * sigmoid(z)
//
// With bf16 tensors y, the gate and the product are each stored in bf16.
//
// It needs the whole row of a token (every head), while the attention
// kernels work one head per workgroup, so it is a pass of its own: one
// workgroup per row, the row held in registers between the sum of squares and
// the scaling, so o and z are read once and out written once (HBM-bound).
#include "sgla_internal.h"

namespace sgla {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements of a row as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T *p, float v[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float v[8]) {
    const u32x4 r = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(r[j] << 16);
        v[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__device__ __forceinline__ void store8(T *p, const float v[8]);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t *p, const float v[8]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 a = (__bf16)v[2 * j], b = (__bf16)v[2 * j + 1];
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4 *>(p));  // not read again here
}
template <>
__device__ __forceinline__ void store8<float>(float *p, const float v[8]) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32x4v{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4v *>(p));
    __builtin_nontemporal_store(f32x4v{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4v *>(p) + 1);
}

template <typename T>
__device__ __forceinline__ float rnd(float x) { return x; }
template <>
__device__ __forceinline__ float rnd<uint16_t>(float x) { return round_bf16(x); }

constexpr int NT = 256;

// NP: pieces of 8 elements per thread (width <= NP * 8 * 256).
template <typename T, int NP>
__global__ __launch_bounds__(NT) void out_norm_gate_kernel(const T *o,  // may equal out
                                                           const T *__restrict__ z,
                                                           const float *__restrict__ w,
                                                           T *out, int width, float eps) {
    const int64_t base = (int64_t)blockIdx.x * width;
    const int tid = threadIdx.x;
    float x[NP][8], zl[NP][8];
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = (p * NT + tid) * 8;
        if (c < width) {
            load8(o + base + c, x[p]);
            load8(z + base + c, zl[p]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(x[p][e], x[p][e], ss);
        }
    }
    // Row sum: within each wave, then across the four waves through LDS.
    __shared__ float part[NT / 64];
    static_assert(sizeof(part) <= kLdsPerCU / 8, "eight workgroups must fit one CU's LDS");
    ss = row16_sum(ss);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    ss = part[0] + part[1] + part[2] + part[3];
    const float rs = rsqrtf(ss / (float)width + eps);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = (p * NT + tid) * 8;
        if (c < width) {
            const float4 w0 = *reinterpret_cast<const float4 *>(w + c);
            const float4 w1 = *reinterpret_cast<const float4 *>(w + c + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = rnd<T>(x[p][e] * rs * wv[e]);
                const float s = rnd<T>(1.f / (1.f + __expf(-zl[p][e])));
                r[e] = y * s;  // rounded by the store for bf16
            }
            store8(out + base + c, r);
        }
    }
}

template <typename T>
hipError_t launch_t(const void *o, const void *z, const float *w, void *out, int64_t rows,
                    int width, float eps, hipStream_t st) {
    const int np = (width + NT * 8 - 1) / (NT * 8);
    const dim3 grid((unsigned)rows), block(NT);
    const T *op = static_cast<const T *>(o);
    const T *zp = static_cast<const T *>(z);
    T *outp = static_cast<T *>(out);
    if (np <= 1) hipLaunchKernelGGL((out_norm_gate_kernel<T, 1>), grid, block, 0, st, op, zp, w, outp, width, eps);
    else if (np <= 2) hipLaunchKernelGGL((out_norm_gate_kernel<T, 2>), grid, block, 0, st, op, zp, w, outp, width, eps);
    else if (np <= 4) hipLaunchKernelGGL((out_norm_gate_kernel<T, 4>), grid, block, 0, st, op, zp, w, outp, width, eps);
    else hipLaunchKernelGGL((out_norm_gate_kernel<T, 8>), grid, block, 0, st, op, zp, w, outp, width, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_out_norm_gate(const void *o, const void *z, const float *w, void *out,
                                int64_t rows, int width, float eps, bool bf16, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (bf16) return launch_t<uint16_t>(o, z, w, out, rows, width, eps, st);
    return launch_t<float>(o, z, w, out, rows, width, eps, st);
}

}  // namespace sgla
