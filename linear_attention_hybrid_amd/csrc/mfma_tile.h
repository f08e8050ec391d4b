// Matrix-core tile helpers shared by the chunked kernels: bf16 32x32x16 MFMA
// with fp32 accumulation, swizzled LDS tile layouts, bf16 packing, the wave
// prefix sum of the gate, direct global-to-LDS loads with their waits,
// range-checked buffer loads and stores, and the transposing LDS read.
// Internal; not part of the ABI.
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

// Eight floats as a bf16 pair hi + lo with |x - hi - lo| < 2^-16 |x|: hi is
// x cut to its top 16 bits (one byte permute per two values), lo the
// remainder, exact in fp32, rounded to bf16.
__device__ __forceinline__ void split_bf16x8(const float *x, bf16x8 &hi, bf16x8 &lo) {
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t a = __float_as_uint(x[2 * e]), b = __float_as_uint(x[2 * e + 1]);
        h[e] = __builtin_amdgcn_perm(b, a, 0x07060302u);
        l[e] = pack_f32(x[2 * e] - __uint_as_float(a & 0xffff0000u),
                        x[2 * e + 1] - __uint_as_float(b & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Eight floats rounded to bf16 (nearest even), two per conversion.
__device__ __forceinline__ bf16x8 to_bf16x8(const float *x) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack_f32(x[2 * e], x[2 * e + 1]);
    return __builtin_bit_cast(bf16x8, r);
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


// ---- Direct global -> LDS loads and the transposing LDS read (gfx950).
//
// global_load_lds_dwordx4: every lane names its own 16-byte global source;
// lane t's data lands at the wave-uniform LDS base (M0) + 16 t (the dword
// form: + 4 t). Written as inline assembly so that the compiler adds no waits
// of its own before later LDS reads (it cannot tell the target buffers apart
// and would wait for every load in flight); callers order them with wait_vm_n.
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
__device__ __forceinline__ void gll16(const void *src, const char *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst))), "v"(src)
                 : "memory", "m0");
}
// The same with the non-temporal hint, for data read once.
__device__ __forceinline__ void gll16_nt(const void *src, const char *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst))), "v"(src)
                 : "memory", "m0");
}
__device__ __forceinline__ void gll4(const void *src, const char *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_dst))), "v"(src)
                 : "memory", "m0");
}

// Wait until at most n (0 .. 63) vector-memory operations of this wave are
// outstanding; they complete in issue order. n must be wave-uniform.
__device__ __forceinline__ void wait_vm_n(int n) {
    switch (n) {
#define SGLA_W(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        SGLA_W(1) SGLA_W(2) SGLA_W(3) SGLA_W(4) SGLA_W(5) SGLA_W(6) SGLA_W(7)
        SGLA_W(8) SGLA_W(9) SGLA_W(10) SGLA_W(11) SGLA_W(12) SGLA_W(13) SGLA_W(14) SGLA_W(15)
        SGLA_W(16) SGLA_W(17) SGLA_W(18) SGLA_W(19) SGLA_W(20) SGLA_W(21) SGLA_W(22) SGLA_W(23)
        SGLA_W(24) SGLA_W(25) SGLA_W(26) SGLA_W(27) SGLA_W(28) SGLA_W(29) SGLA_W(30) SGLA_W(31)
        SGLA_W(32) SGLA_W(33) SGLA_W(34) SGLA_W(35) SGLA_W(36) SGLA_W(37) SGLA_W(38) SGLA_W(39)
        SGLA_W(40) SGLA_W(41) SGLA_W(42) SGLA_W(43) SGLA_W(44) SGLA_W(45) SGLA_W(46) SGLA_W(47)
        SGLA_W(48) SGLA_W(49) SGLA_W(50) SGLA_W(51) SGLA_W(52) SGLA_W(53) SGLA_W(54) SGLA_W(55)
        SGLA_W(56) SGLA_W(57) SGLA_W(58) SGLA_W(59) SGLA_W(60) SGLA_W(61) SGLA_W(62) SGLA_W(63)
#undef SGLA_W
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// A raw buffer resource over [base, base + bytes): the hardware's range check
// makes loads past the end return zeros and drops stores past the end, so a
// ragged tile needs no branch around its loads and stores. Word 3 selects
// 32-bit data, which the untyped loads and stores of gfx9-family chips need.
// bytes < 2^31; offsets are unsigned 32-bit.
typedef __amdgpu_buffer_rsrc_t buf_t;
__device__ __forceinline__ buf_t buf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(buf_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// Non-temporal load (the nt bit), for data that nothing reads again.
__device__ __forceinline__ u32x4 buf_ld16_nt(buf_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
__device__ __forceinline__ float buf_ld_f32(buf_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_st16(buf_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
// Non-temporal store (the nt bit): for outputs that nothing in the same call
// reads again, so that they do not push the call's re-read data out of the
// caches.
__device__ __forceinline__ void buf_st16_nt(buf_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 2);
}
__device__ __forceinline__ void buf_st8(buf_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}

// A use of x that the compiler cannot see through, so it waits for x's load
// here. Used before a loop so that the loop's own waits need not cover loads
// from before it. x is a scalar or a 16-byte vector (the host pass parses the
// constraint too).
template <typename T>
__device__ __forceinline__ void settle(const T &x) { asm volatile("" ::"v"(x)); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8 bytes named by lane 4k + i / 4, for k = 0..3. With lane m of
// the group naming row r0 + m / 4, columns c0 + 4 (m % 4) .. + 3 of a
// row-major bf16 tile, lane i gets column c0 + i of rows r0 .. r0 + 3: four
// consecutive rows of one column, as an MFMA operand needs them.
typedef short sgla_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr(const char *lds, int off) {
    const sgla_v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) sgla_v4s *)((__attribute__((address_space(3))) char *)(lds + off)));
    return __builtin_bit_cast(bf16x4, r);
}

// Byte offset, in a 64 x 128 bf16 row tile swizzled as row_off, of the 8 bytes
// lane m of a 16-lane group names for the transposing read of rows r0 .. r0+3,
// columns c0 .. c0+15 (r0 a multiple of 4, c0 a multiple of 16).
__device__ __forceinline__ int tr_src(int r0, int c0, int m) {
    const int r = r0 + (m >> 2);
    const int cc = (c0 >> 3) + ((m & 3) >> 1);
    return r * 256 + ((cc ^ (r & 15)) << 4) + 8 * (m & 1);
}

}  // namespace sgla
