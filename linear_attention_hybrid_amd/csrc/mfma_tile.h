// Matrix-core tile helpers shared by the chunked kernels: bf16 32x32x16 MFMA
// with fp32 accumulation, swizzled LDS tile layouts, bf16 packing and the
// wave prefix sum of the gate. Internal; not part of the ABI.
//
// MFMA 32x32x16 register layout (v_mfma_f32_32x32x16_bf16): for D = A B + C,
// lane l supplies A[l % 32][8 (l / 32) .. + 7] and B[8 (l / 32) .. + 7][l % 32]
// (eight bf16 each) and holds D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32] in
// accumulator element v. The order of the sixteen k values inside one
// instruction is free as long as A and B agree on it, which the kernels use to
// feed an accumulator straight back in as an operand.
#pragma once

#include "sgla_internal.h"

namespace sgla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte offset of 16-byte chunk c of row r in a 256-byte-row tile (64 x 128 bf16).
__device__ __forceinline__ int row_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
// Byte offset of 16-byte chunk c (8 tokens) of row d in a 128-byte-row tile (128 x 64 bf16).
__device__ __forceinline__ int tr_off(int d, int c) {
    return d * 128 + ((c ^ (((d >> 1) ^ (d >> 3)) & 7)) << 4);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_f32(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T lds_ld(const char *lds, int off) {
    return *reinterpret_cast<const T *>(lds + off);
}
template <typename T>
__device__ __forceinline__ void lds_st(char *lds, int off, T v) {
    *reinterpret_cast<T *>(lds + off) = v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts inside
// each 16-lane row, then the row totals carried by row broadcasts (lanes with
// no source lane add zero).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    int v = __builtin_bit_cast(int, x);
#define SGLA_DPP_ADD(ctrl, rmask)                                                          \
    v = __builtin_bit_cast(int, __builtin_bit_cast(float, v) +                              \
                                    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp( \
                                        0, v, ctrl, rmask, 0xf, false)))
    SGLA_DPP_ADD(0x111, 0xf);  // row_shr:1
    SGLA_DPP_ADD(0x112, 0xf);  // row_shr:2
    SGLA_DPP_ADD(0x114, 0xf);  // row_shr:4
    SGLA_DPP_ADD(0x118, 0xf);  // row_shr:8
    SGLA_DPP_ADD(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    SGLA_DPP_ADD(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef SGLA_DPP_ADD
    return __builtin_bit_cast(float, v);
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

}  // namespace sgla
