// Internal declarations shared by the libsgla HIP sources. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgla {

constexpr int kChunk = 64;  // tokens per chunk (the chunk size the pages use)
// LDS of one gfx950 compute unit, shared by the workgroups resident on it.
// Every kernel states its footprint against this with a static_assert, times
// the workgroups per CU it is built to run with.
constexpr int kLdsPerCU = 160 * 1024;

// One segment of one sequence: a run of whole chunks handled by one
// workgroup column. Built on the device from cu_seqlens (or from B x T).
struct SegEntry {
    int64_t tok0;  // packed index of the segment's first token
    int32_t len;   // tokens in the segment; -1 marks an unused table row
    int32_t seq;   // sequence index
    int32_t p;     // segment index inside its sequence
    int32_t nseg;  // number of segments of that sequence
    int32_t pad0;
    int32_t pad1;
};
static_assert(sizeof(SegEntry) == 32, "SegEntry layout");

struct SeqEntry {
    int32_t first;  // table row of the sequence's first segment
    int32_t nseg;   // number of segments (>= 1, also for empty sequences)
};

// Arguments of the chunked-forward kernels.
struct ChunkParams {
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const float *s0;      // [N,H,Dk,Dv] or nullptr
    void *out;
    float *sfin;          // [N,H,Dk,Dv] or nullptr
    float *buf;           // [nseg_max,H,Dk,Dv]: segment states, then carried-in states
    float *gam;           // [nseg_max,H]: total log-decay of each segment
    const SegEntry *segs;  // [nseg_max], or nullptr: arithmetic segments (see seg_at)
    const SeqEntry *seqs;  // [N], or nullptr likewise
    // Packed sequences without a table: one segment per sequence, read from
    // the offsets (segs == nullptr; nps == 1; T is the packed total).
    const int64_t *cu;
    int H;
    int nseg_max;
    int N;
    float scale;
    int T;        // tokens per sequence when segs == nullptr
    int seg_len;  // tokens per segment (a multiple of the chunk size)
    int nps;      // segments per sequence when segs == nullptr
    // q/k prologue (per-head RMSNorm, then rotate-half RoPE) applied as the
    // tiles are loaded; qw == nullptr: none.
    const float *qw;         // [Dk] RMSNorm weight of q
    const float *kw;         // [Dk] RMSNorm weight of k
    const int32_t *pos_off;  // [N] position of each sequence's first token, or nullptr (0)
    float theta;             // RoPE base
    float eps;               // RMSNorm epsilon
    // Sub-segments per output segment: the state and scan kernels work on
    // segments of seg_len tokens, and an output pass over segments rsub times
    // longer starts output segment j of a sequence from the state the scan
    // leaves in slot first + rsub * j. 1 when both passes use the same segments.
    int rsub;
    // Nonzero: the state pass (without the prologue) runs one workgroup per
    // (sub-segment, head, half of the value columns) instead of one per
    // (sub-segment, head).
    int state_halves;
};

// Arguments of the value-half output kernel (chunk_halves.hip): the output
// segments (oseg_len tokens each, from `osegs` or arithmetic), and in `c` the
// sub-segment tables, the state buffer and the tensors.
struct HalvesParams {
    ChunkParams c;
    const SegEntry *osegs;  // [onseg_max], or nullptr for B equal rows
    int onseg_max;
    int onps;               // output segments per sequence when osegs == nullptr
    int oseg_len;           // tokens per output segment (a multiple of the chunk size)
};

// Sequence n of a packed call as one segment, straight from the offsets;
// offsets that break the documented rule are clamped into [0, T].
__device__ __forceinline__ SegEntry seg_from_cu(const int64_t *cu, int n, int T) {
    int64_t a = cu[n], b = cu[n + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    SegEntry e;
    e.tok0 = a;
    e.len = (int32_t)(b - a);
    e.seq = n;
    e.p = 0;
    e.nseg = 1;
    e.pad0 = 0;
    e.pad1 = 0;
    return e;
}

// Segment s of the call. Without a table every sequence has the same T
// tokens and nps segments, so the entry is arithmetic (or, for packed
// sequences, the whole sequence s).
__device__ __forceinline__ SegEntry seg_at(const ChunkParams &p, int s) {
    if (p.segs) return p.segs[s];
    if (p.cu) return seg_from_cu(p.cu, s, p.T);
    SegEntry e;
    const int n = s / p.nps;
    const int j = s - n * p.nps;
    e.seq = n;
    e.p = j;
    e.nseg = p.nps;
    e.tok0 = (int64_t)n * p.T + (int64_t)j * p.seg_len;
    const int rem = p.T - j * p.seg_len;
    e.len = rem < p.seg_len ? rem : p.seg_len;
    e.pad0 = 0;
    e.pad1 = 0;
    return e;
}

__device__ __forceinline__ SeqEntry seq_at(const ChunkParams &p, int n) {
    if (p.seqs) return p.seqs[n];
    if (p.cu) return SeqEntry{n, 1};
    SeqEntry e;
    e.first = n * p.nps;
    e.nseg = p.nps;
    return e;
}

// ---- q/k prologue helpers (page "MiniCPM-SALA — Complete Blueprint",
// section "B2 lightning-attn (Simple GLA)": per-head RMSNorm of q and k with
// one weight vector of length Dk, stored in bf16; then RoPE with base theta
// on the fp32 values, stored in bf16). RoPE turns the pair (i, i + Dk/2) by
// pos * theta^(-2i/Dk) radians in the positive sense:
// (a, b) -> (a cos - b sin, b cos + a sin).

// Round to the nearest bf16 (ties to even) and back to fp32.
__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

// Turns per position of frequency i: theta^(-2i/dk) / (2 pi), in fp64.
__device__ __forceinline__ double rope_turns_per_pos(int i, int dk, float theta) {
    return exp2(-(2.0 * i / dk) * log2((double)theta)) * 0.15915494309189533577;
}

// Fractional turns of pos * omega, reduced in fp64 so that positions up to
// 2^31 keep about 1e-7 turn of accuracy; the result lies in [-0.5, 0.5].
__device__ __forceinline__ float rope_base_turns(int64_t pos, double turns_per_pos) {
    double t = (double)pos * turns_per_pos;
    return (float)(t - rint(t));
}

// sin and cos of an angle given in turns (|x| < 256): the hardware
// instructions take turns directly.
__device__ __forceinline__ float sin_turns(float x) { return __builtin_amdgcn_sinf(x); }
__device__ __forceinline__ float cos_turns(float x) { return __builtin_amdgcn_cosf(x); }

// Sum over the 16 lanes of a DPP row (lanes 16a .. 16a+15), in every lane:
// rotations by 8, 4, 2, 1 inside the row.
__device__ __forceinline__ float row16_sum(float x) {
#define SGLA_ROR_ADD(ctrl) \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false))
    SGLA_ROR_ADD(0x128);  // row_ror:8
    SGLA_ROR_ADD(0x124);  // row_ror:4
    SGLA_ROR_ADD(0x122);  // row_ror:2
    SGLA_ROR_ADD(0x121);  // row_ror:1
#undef SGLA_ROR_ADD
    return x;
}

// The value lane (l ^ 8) holds, for lanes of one DPP row (rotation by 8).
// No `old` operand, so the move can fold into the instruction that uses it.
__device__ __forceinline__ float row16_swap8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf, true));
}

// Arguments of the chunked gated-delta-rule kernels. The chunk table is the
// segment table with one chunk per segment (seg_len = kChunk).
struct GdnParams {
    ChunkParams c;      // q, k, v, g, s0, out, sfin, segs, seqs, H, nseg_max, N, scale, T, nps
    const float *beta;  // [tokens, H] write strength of each token
    char *tiles;        // [nseg_max, H] tiles of 48 KiB: W rows (bf16) and U^T (fp32) of each
                        // chunk; U's slices later hold the chunk's start state for the output
    char *nvimg;        // [nseg_max, H] 16 KiB: each chunk's new_v for the output
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_plan(const int64_t *cu, int B, int T, int seg_len, int nseg_max,
                       SegEntry *segs, SeqEntry *seqs, hipStream_t st);
hipError_t launch_scan(const ChunkParams &p, int Dk, int Dv, hipStream_t st);
// Writes to *status the bits of the rules cu_seqlens breaks (0: none):
// 1 cu[0] != 0, 2 some cu[i] > cu[i+1], 4 cu[B] != T.
hipError_t launch_validate_cu(const int64_t *cu, int B, int T, int32_t *status, hipStream_t st);
hipError_t launch_chunk_valu(const ChunkParams &p, bool bf16, int Dk, int Dv, bool phase_state,
                             hipStream_t st);
hipError_t launch_chunk_mfma(const ChunkParams &p, bool phase_state, hipStream_t st);
hipError_t launch_chunk_halves(const HalvesParams &hp, hipStream_t st);
hipError_t launch_qk_norm_rope(const void *x, const float *w, const int32_t *pos_off, void *out,
                               int B, int T, int H, float theta, float eps, hipStream_t st);
hipError_t launch_out_norm_gate(const void *o, const void *z, const float *w, void *out,
                                int64_t rows, int width, float eps, bool bf16, hipStream_t st);
// Decode-step prologue arguments; qw == nullptr: none.
struct StepPrologue {
    const float *qw;
    const float *kw;
    const int32_t *pos;  // [N] position of each row's token
    float theta;
    float eps;
};
hipError_t launch_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                 void *state, bool state_bf16, const int32_t *idx, void *out,
                                 int N, int H, int Dk, int Dv, float scale, bool bf16,
                                 const StepPrologue &pro, hipStream_t st);

hipError_t launch_gdn_chunk(const GdnParams &p, hipStream_t st);

// Arguments of the chunked KDA kernels (kda_chunk.hip): the chunk table is
// the segment table with one chunk per segment, as for GDN; g is [tokens, H,
// Dk].
struct KdaParams {
    ChunkParams c;      // q, k, v, g, s0, out, sfin, segs, seqs, H, nseg_max, N, scale, T, nps
    const float *beta;  // [tokens, H]
    float *tiles;       // [nseg_max, H] of 2 * 64 * Dk + 64 * Dv + Dk floats: W, K * exp(G_last - G), U, exp(G_last)
    float *nv;          // [nseg_max, H, 64, Dv] new_v of each chunk
    float *sin;         // [nseg_max, H, Dk, Dv] start state of each chunk
    int dk, dv;
};
// Workspace bytes per (chunk, head) of the chunked KDA kernels.
size_t kda_chunk_bytes(int dk, int dv);
hipError_t launch_kda_chunk(const KdaParams &p, bool bf16, hipStream_t st);
// per_dim_gate: g is [N, H, Dk] (KDA), else [N, H].
hipError_t launch_gdn_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, const int32_t *idx, void *out, int N,
                           int H, int Dk, int Dv, float scale, bool bf16, bool per_dim_gate,
                           hipStream_t st);

// Map a linear workgroup id onto (unit, sub) so that the `nsub` workgroups of
// one unit land on the same XCD (ids are dealt to the 8 XCDs round-robin) and
// are dispatched close together, so they share that XCD's L2.
__device__ __forceinline__ void xcd_unit_map(int id, int nsub, int &unit, int &sub) {
    const int xcd = id & 7;
    const int j = id >> 3;
    unit = (j / nsub) * 8 + xcd;
    sub = j % nsub;
}

// bf16 <-> fp32 (round to nearest even on the way down; NaN kept quiet).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void store_elem(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float x) {
    p[i] = f32_to_bf16(x);
}

}  // namespace sgla
