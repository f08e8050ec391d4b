// Host side of the libsgla C ABI: argument checks, planning, launches.
#include <stdlib.h>
#include <string.h>

#include "../../include/sgla.h"
#include "sgla_internal.h"

using namespace sgla;

namespace {

constexpr int kVersion = 100;  // 0.1.0
// Heads per call: keeps the byte offset of a token row inside a 64-token
// chunk (64 * H * Dv * 2 bytes) within 32 bits.
constexpr int kMaxHeads = 65536;
// Widest row of the output epilogue: the kernel keeps a row in registers,
// up to 8 pieces of 8 elements per thread of a 256-thread workgroup.
constexpr int kMaxOutWidth = 16384;

bool misaligned(const void *p, uintptr_t a = 16) {
    return p && (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}
bool head_size_ok(int d) { return d == 64 || d == 128; }

// Tokens per segment for the chunked forward: long enough that per-segment
// state traffic (one Dk x Dv fp32 state written, scanned and re-read per
// segment) stays small next to the token traffic, short enough that the number
// of (segment, head) units keeps every compute unit busy.
int choose_seg_len(int64_t ttot, int B, int H) {
    const char *env = getenv("SGLA_SEG_LEN");
    if (env) {
        long v = strtol(env, nullptr, 10);
        if (v >= kChunk && v % kChunk == 0 && v <= (1 << 24)) return (int)v;
    }
    const int64_t target_units = 2048;  // about 8 per compute unit
    int64_t len = (ttot * H + target_units - 1) / target_units;
    if (len < 512) len = 512;
    if (len > 8192) len = 8192;
    len = (len + kChunk - 1) / kChunk * kChunk;
    (void)B;
    return (int)len;
}

// Output segments of the value-half kernel (bf16, 128-wide heads): long
// enough that two workgroups per compute unit cover the call, two per
// (segment, head), and at least 512 tokens.
int choose_out_len(int64_t ttot, int H) {
    const char *env = getenv("SGLA_OUT_SEG_LEN");
    if (env) {
        long v = strtol(env, nullptr, 10);
        if (v >= kChunk && v % kChunk == 0 && v <= (1 << 24)) return (int)v;
    }
    const int64_t target_wgs = 512;
    int64_t len = (ttot * H * 2 + target_wgs - 1) / target_wgs;
    if (len < 512) len = 512;
    if (len > (1 << 24)) len = 1 << 24;
    return (int)((len + kChunk - 1) / kChunk * kChunk);
}

// Sub-segments per output segment for the state pass: split until the pass
// has about 384 (segment, head) workgroups, keeping sub-segments of at least
// 512 tokens and whole chunks. pre_units = (segment, head) pairs whose state
// is needed when each output segment is one sub-segment.
int choose_rsub(int out_len, int64_t pre_units) {
    const char *env = getenv("SGLA_RSUB");
    if (env) {
        long v = strtol(env, nullptr, 10);
        if (v >= 1 && v <= out_len / kChunk && (out_len / kChunk) % v == 0) return (int)v;
    }
    int r = 1;
    while (out_len / (2 * r) >= 512 && (out_len / kChunk) % (2 * r) == 0 && pre_units * r < 384) r *= 2;
    return r;
}

sgla_status hip_status(hipError_t e) { return e == hipSuccess ? SGLA_OK : SGLA_ERR_HIP; }

// Arguments of the q/k prologue (RMSNorm, RoPE) as the entry points get them.
struct ProArgs {
    const float *qw;
    const float *kw;
    const int32_t *pos;  // chunked forward: per-sequence offsets (may be null); step: per row
    float theta;
    float eps;
};

bool finite(float x) { return x == x && x - x == 0.f; }

sgla_status check_prologue(const ProArgs &a) {
    if (!a.qw || !a.kw) return SGLA_ERR_INVALID_ARG;
    if (misaligned(a.qw, 4) || misaligned(a.kw, 4) || misaligned(a.pos, 4)) return SGLA_ERR_INVALID_ARG;
    if (!finite(a.theta) || !(a.theta > 0.f) || !finite(a.eps) || a.eps < 0.f)
        return SGLA_ERR_INVALID_ARG;
    return SGLA_OK;
}

sgla_status chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, void *out, float *final_state,
                      const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv, float scale,
                      sgla_dtype dtype, void *stream, const ProArgs *pro);
sgla_status chunk_fwd_halves(const void *q, const void *k, const void *v, const float *g,
                             const float *initial_state, void *out, float *final_state,
                             const int64_t *cu_seqlens, int B, int T, int H, float scale,
                             void *stream);

}  // namespace

extern "C" {

const char *sgla_status_string(sgla_status s) {
    switch (s) {
        case SGLA_OK: return "SGLA_OK";
        case SGLA_ERR_INVALID_ARG: return "SGLA_ERR_INVALID_ARG";
        case SGLA_ERR_UNSUPPORTED: return "SGLA_ERR_UNSUPPORTED";
        case SGLA_ERR_HIP: return "SGLA_ERR_HIP";
    }
    return "SGLA_ERR_UNKNOWN";
}

int sgla_version(void) { return kVersion; }

sgla_status sgla_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                           const float *initial_state, void *out, float *final_state,
                           const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                           float scale, sgla_dtype dtype, void *stream) {
    return chunk_fwd(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H, Dk, Dv,
                     scale, dtype, stream, nullptr);
}

sgla_status sgla_chunk_fwd_qk_norm_rope(const void *q, const void *k, const void *v,
                                        const float *g, const float *initial_state, void *out,
                                        float *final_state, const int64_t *cu_seqlens,
                                        const float *q_weight, const float *k_weight,
                                        const int32_t *pos_offset, float theta, float eps, int B,
                                        int T, int H, int Dk, int Dv, float scale,
                                        sgla_dtype dtype, void *stream) {
    const ProArgs pro{q_weight, k_weight, pos_offset, theta, eps};
    return chunk_fwd(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H, Dk, Dv,
                     scale, dtype, stream, &pro);
}

}  // extern "C"

namespace {

sgla_status chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, void *out, float *final_state,
                      const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv, float scale,
                      sgla_dtype dtype, void *stream, const ProArgs *pro) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    if (!head_size_ok(Dk) || !head_size_ok(Dv)) return SGLA_ERR_UNSUPPORTED;
    if (H > kMaxHeads) return SGLA_ERR_UNSUPPORTED;
    if (pro) {
        // The prologue is built into the bf16 matrix-core kernels (128-wide heads).
        if (dtype != SGLA_BF16 || Dk != 128 || Dv != 128) return SGLA_ERR_UNSUPPORTED;
        const sgla_status ps = check_prologue(*pro);
        if (ps != SGLA_OK) return ps;
    }
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    if ((int64_t)B * H > (int64_t)1 << 30) return SGLA_ERR_INVALID_ARG;
    if (ttot > 0 && (!q || !k || !v || !g || !out)) return SGLA_ERR_INVALID_ARG;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g, 4) || misaligned(out) ||
        misaligned(initial_state) || misaligned(final_state) || misaligned(cu_seqlens, 8))
        return SGLA_ERR_INVALID_ARG;
    if (B == 0) return SGLA_OK;
    if (ttot == 0 && !final_state) return SGLA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);

    // bf16 with 128-wide heads and no prologue: equal-length batches run on
    // the value-half kernels (less state traffic; as fast on 8K-token
    // sequences and faster on long ones). Packed sequences of mixed lengths
    // stay on the one-level kernels, whose shorter segments balance better:
    // there the per-chunk work bounds the call, and the value halves repeat
    // the scores. SGLA_VALUE_HALVES / SGLA_ONE_LEVEL force either path.
    const bool bf16 = dtype == SGLA_BF16;
    const bool halves = cu_seqlens ? getenv("SGLA_VALUE_HALVES") != nullptr
                                   : getenv("SGLA_ONE_LEVEL") == nullptr;
    if (bf16 && Dk == 128 && Dv == 128 && !pro && !getenv("SGLA_FORCE_VALU") && halves)
        return chunk_fwd_halves(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H,
                                scale, stream);

    const int seg_len = choose_seg_len(ttot, B, H);
    // Without cu_seqlens every sequence has T tokens and the same number of
    // segments, so no table is built; with it, a device-side plan kernel lays
    // the segments out (the host never reads the offsets).
    const bool table = cu_seqlens != nullptr;
    const int64_t nps64 = T == 0 ? 1 : ((int64_t)T + seg_len - 1) / seg_len;
    const int64_t nseg_max64 = table ? ttot / seg_len + B + 1 : (int64_t)B * nps64;
    // The vector-ALU kernels run one workgroup per 32 value columns of each
    // (segment, head); every grid must stay below 2^31.
    if (nseg_max64 * H * ((Dv + 31) / 32) > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    const int nseg_max = (int)nseg_max64;
    // Sequences that fit in one segment need no segment states and no scan.
    const bool split = table || nps64 > 1;

    // Workspace: segment table, sequence table, per-segment log-decays, states.
    const size_t segs_b = table ? (size_t)nseg_max * sizeof(SegEntry) : 0;
    const size_t seqs_b = table ? ((size_t)B * sizeof(SeqEntry) + 255) / 256 * 256 : 0;
    const size_t gam_b = split ? ((size_t)nseg_max * H * sizeof(float) + 255) / 256 * 256 : 0;
    const size_t buf_b = split ? (size_t)nseg_max * H * Dk * Dv * sizeof(float) : 0;
    const size_t ws_b = segs_b + seqs_b + gam_b + buf_b;
    char *ws = nullptr;
    hipError_t e = hipSuccess;
    if (ws_b) {
        e = hipMallocAsync(reinterpret_cast<void **>(&ws), ws_b, st);
        if (e != hipSuccess) return SGLA_ERR_HIP;
    }

    ChunkParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.s0 = initial_state;
    p.out = out;
    p.sfin = final_state;
    p.segs = table ? reinterpret_cast<SegEntry *>(ws) : nullptr;
    p.seqs = table ? reinterpret_cast<SeqEntry *>(ws + segs_b) : nullptr;
    p.gam = split ? reinterpret_cast<float *>(ws + segs_b + seqs_b) : nullptr;
    p.buf = split ? reinterpret_cast<float *>(ws + segs_b + seqs_b + gam_b) : nullptr;
    p.H = H;
    p.nseg_max = nseg_max;
    p.N = B;
    p.scale = scale;
    p.T = T;
    p.seg_len = seg_len;
    p.nps = (int)nps64;
    p.qw = pro ? pro->qw : nullptr;
    p.kw = pro ? pro->kw : nullptr;
    p.pos_off = pro ? pro->pos : nullptr;
    p.theta = pro ? pro->theta : 0.f;
    p.eps = pro ? pro->eps : 0.f;
    p.rsub = 1;

    // bf16 with 128-wide heads runs on the matrix cores; every other
    // combination on the vector ALUs.
    const bool mfma = bf16 && Dk == 128 && Dv == 128 && (pro || !getenv("SGLA_FORCE_VALU"));
    auto phase = [&](bool state_phase) {
        return mfma ? launch_chunk_mfma(p, state_phase, st)
                    : launch_chunk_valu(p, bf16, Dk, Dv, state_phase, st);
    };
    if (table)
        e = launch_plan(cu_seqlens, B, T, seg_len, nseg_max, reinterpret_cast<SegEntry *>(ws),
                        reinterpret_cast<SeqEntry *>(ws + segs_b), st);
    if (e == hipSuccess && split) e = phase(/*state_phase=*/true);
    if (e == hipSuccess && split) e = launch_scan(p, Dk, Dv, st);
    if (e == hipSuccess) e = phase(/*state_phase=*/false);
    if (ws) {
        const hipError_t ef = hipFreeAsync(ws, st);
        if (e == hipSuccess) e = ef;
    }
    return hip_status(e);
}

// bf16, Dk = Dv = 128, no prologue: output segments of oseg_len tokens over
// value-column halves (chunk_halves.hip). When a sequence spans several
// output segments, the state kernel first computes the zero-start state of
// every sub-segment (oseg_len / rsub tokens) that precedes its last output
// segment, and the scan turns them into the start state of each output
// segment. Arguments are checked by chunk_fwd.
sgla_status chunk_fwd_halves(const void *q, const void *k, const void *v, const float *g,
                             const float *initial_state, void *out, float *final_state,
                             const int64_t *cu_seqlens, int B, int T, int H, float scale,
                             void *stream) {
    constexpr int D = 128;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool table = cu_seqlens != nullptr;
    const int64_t ttot = table ? (int64_t)T : (int64_t)B * T;
    const int oseg_len = choose_out_len(ttot, H);
    const int64_t onps64 = T == 0 ? 1 : ((int64_t)T + oseg_len - 1) / oseg_len;
    const int64_t onseg64 = table ? ttot / oseg_len + B + 1 : (int64_t)B * onps64;
    if (onseg64 * H * 2 > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    const bool split = table || onps64 > 1;
    const int64_t pre_units = table ? (ttot / oseg_len) * H : (onps64 - 1) * B * H;
    const int rsub = split ? choose_rsub(oseg_len, pre_units) : 1;
    const int sub_len = oseg_len / rsub;
    const int64_t nps64 = T == 0 ? 1 : ((int64_t)T + sub_len - 1) / sub_len;
    const int64_t nseg64 = !split ? 0 : table ? ttot / sub_len + B + 1 : (int64_t)B * nps64;
    if (nseg64 * H > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;

    // Workspace: output-segment table, sub-segment tables, log-decays, states.
    auto r256 = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t osegs_b = table ? r256((size_t)onseg64 * sizeof(SegEntry)) : 0;
    const size_t oseqs_b = table ? r256((size_t)B * sizeof(SeqEntry)) : 0;
    const size_t segs_b = table ? r256((size_t)nseg64 * sizeof(SegEntry)) : 0;
    const size_t seqs_b = table ? r256((size_t)B * sizeof(SeqEntry)) : 0;
    const size_t gam_b = split ? r256((size_t)nseg64 * H * sizeof(float)) : 0;
    const size_t buf_b = split ? (size_t)nseg64 * H * D * D * sizeof(float) : 0;
    const size_t ws_b = osegs_b + oseqs_b + segs_b + seqs_b + gam_b + buf_b;
    char *ws = nullptr;
    hipError_t e = hipSuccess;
    if (ws_b) {
        e = hipMallocAsync(reinterpret_cast<void **>(&ws), ws_b, st);
        if (e != hipSuccess) return SGLA_ERR_HIP;
    }
    char *wp = ws;
    auto take = [&](size_t b) { char *r = b ? wp : nullptr; wp += b; return r; };
    SegEntry *osegs = reinterpret_cast<SegEntry *>(take(osegs_b));
    SeqEntry *oseqs = reinterpret_cast<SeqEntry *>(take(oseqs_b));
    SegEntry *segs = reinterpret_cast<SegEntry *>(take(segs_b));
    SeqEntry *seqs = reinterpret_cast<SeqEntry *>(take(seqs_b));
    float *gam = reinterpret_cast<float *>(take(gam_b));
    float *buf = reinterpret_cast<float *>(take(buf_b));

    HalvesParams hp{};
    ChunkParams &p = hp.c;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.s0 = initial_state;
    p.out = out;
    p.sfin = final_state;
    p.buf = buf;
    p.gam = gam;
    p.segs = segs;
    p.seqs = seqs;
    p.H = H;
    p.nseg_max = (int)nseg64;
    p.N = B;
    p.scale = scale;
    p.T = T;
    p.seg_len = sub_len;
    p.nps = (int)nps64;
    p.rsub = rsub;
    hp.osegs = osegs;
    hp.onseg_max = (int)onseg64;
    hp.onps = (int)onps64;
    hp.oseg_len = oseg_len;

    if (table) {
        e = launch_plan(cu_seqlens, B, T, oseg_len, (int)onseg64, osegs, oseqs, st);
        if (e == hipSuccess) e = launch_plan(cu_seqlens, B, T, sub_len, (int)nseg64, segs, seqs, st);
    }
    if (e == hipSuccess && split) e = launch_chunk_mfma(p, /*phase_state=*/true, st);
    if (e == hipSuccess && split) e = launch_scan(p, D, D, st);
    if (e == hipSuccess) e = launch_chunk_halves(hp, st);
    if (ws) {
        const hipError_t ef = hipFreeAsync(ws, st);
        if (e == hipSuccess) e = ef;
    }
    return hip_status(e);
}

sgla_status recurrent_step(const void *q, const void *k, const void *v, const float *g,
                           void *state, sgla_dtype state_dtype, const int32_t *state_indices,
                           void *out, int N, int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                           void *stream, const ProArgs *pro) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (state_dtype != SGLA_F32 && state_dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    if (!head_size_ok(Dk) || !head_size_ok(Dv)) return SGLA_ERR_UNSUPPORTED;
    if (pro) {
        if (dtype != SGLA_BF16 || Dk != 128) return SGLA_ERR_UNSUPPORTED;
        const sgla_status ps = check_prologue(*pro);
        if (ps != SGLA_OK) return ps;
    }
    if ((int64_t)N * H > ((int64_t)1 << 31) - 1) return SGLA_ERR_INVALID_ARG;
    if (N == 0) return SGLA_OK;
    if (!q || !k || !v || !g || !state || !out) return SGLA_ERR_INVALID_ARG;
    if (pro && !pro->pos) return SGLA_ERR_INVALID_ARG;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g, 4) ||
        misaligned(state) || misaligned(out) || misaligned(state_indices, 4))
        return SGLA_ERR_INVALID_ARG;
    StepPrologue sp{};
    if (pro) sp = StepPrologue{pro->qw, pro->kw, pro->pos, pro->theta, pro->eps};
    return hip_status(launch_recurrent_step(q, k, v, g, state, state_dtype == SGLA_BF16,
                                            state_indices, out, N, H, Dk, Dv, scale,
                                            dtype == SGLA_BF16, sp,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

sgla_status sgla_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                float *state, const int32_t *state_indices, void *out, int N,
                                int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                void *stream) {
    return recurrent_step(q, k, v, g, state, SGLA_F32, state_indices, out, N, H, Dk, Dv, scale,
                          dtype, stream, nullptr);
}

sgla_status sgla_recurrent_step_qk_norm_rope(const void *q, const void *k, const void *v,
                                             const float *g, float *state,
                                             const int32_t *state_indices, void *out,
                                             const float *q_weight, const float *k_weight,
                                             const int32_t *positions, float theta, float eps,
                                             int N, int H, int Dk, int Dv, float scale,
                                             sgla_dtype dtype, void *stream) {
    const ProArgs pro{q_weight, k_weight, positions, theta, eps};
    return recurrent_step(q, k, v, g, state, SGLA_F32, state_indices, out, N, H, Dk, Dv, scale,
                          dtype, stream, &pro);
}

sgla_status sgla_recurrent_step_ex(const void *q, const void *k, const void *v, const float *g,
                                   void *state, sgla_dtype state_dtype,
                                   const int32_t *state_indices, void *out,
                                   const float *q_weight, const float *k_weight,
                                   const int32_t *positions, float theta, float eps, int N, int H,
                                   int Dk, int Dv, float scale, sgla_dtype dtype, void *stream) {
    const ProArgs pro{q_weight, k_weight, positions, theta, eps};
    return recurrent_step(q, k, v, g, state, state_dtype, state_indices, out, N, H, Dk, Dv, scale,
                          dtype, stream, q_weight ? &pro : nullptr);
}

sgla_status sgla_out_norm_gate(const void *o, const void *z, const float *weight, void *out,
                               int64_t rows, int width, float eps, sgla_dtype dtype,
                               void *stream) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (rows < 0 || width < 1 || rows > ((int64_t)1 << 31) - 1) return SGLA_ERR_INVALID_ARG;
    if (!finite(eps) || eps < 0.f) return SGLA_ERR_INVALID_ARG;
    if (width % 8 != 0 || width > kMaxOutWidth) return SGLA_ERR_UNSUPPORTED;
    if (rows == 0) return SGLA_OK;
    if (!o || !z || !weight || !out) return SGLA_ERR_INVALID_ARG;
    if (misaligned(o) || misaligned(z) || misaligned(weight) || misaligned(out))
        return SGLA_ERR_INVALID_ARG;
    return hip_status(launch_out_norm_gate(o, z, weight, out, rows, width, eps,
                                           dtype == SGLA_BF16, static_cast<hipStream_t>(stream)));
}

sgla_status sgla_gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, void *out,
                               float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                               int Dk, int Dv, float scale, sgla_dtype dtype, void *stream) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    // The delta rule runs on the bf16 matrix-core kernels with 128-wide heads.
    if (dtype != SGLA_BF16 || Dk != 128 || Dv != 128) return SGLA_ERR_UNSUPPORTED;
    if (H > kMaxHeads) return SGLA_ERR_UNSUPPORTED;
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    if ((int64_t)B * H > (int64_t)1 << 30) return SGLA_ERR_INVALID_ARG;
    // The chain kernel runs eight workgroups per (sequence, head), their count
    // rounded up to a multiple of 64; the grid must stay below 2^31.
    if ((int64_t)B * H > ((int64_t)1 << 28) - 8) return SGLA_ERR_UNSUPPORTED;
    if (ttot > 0 && (!q || !k || !v || !g || !beta || !out)) return SGLA_ERR_INVALID_ARG;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g, 4) ||
        misaligned(beta, 4) || misaligned(out) || misaligned(initial_state) ||
        misaligned(final_state) || misaligned(cu_seqlens, 8))
        return SGLA_ERR_INVALID_ARG;
    if (B == 0) return SGLA_OK;
    if (ttot == 0 && !final_state) return SGLA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);

    // One table row per chunk: without cu_seqlens the rows are arithmetic,
    // with it the plan kernel lays them out on the device.
    const bool table = cu_seqlens != nullptr;
    const int64_t nps64 = T == 0 ? 1 : ((int64_t)T + kChunk - 1) / kChunk;
    const int64_t nch64 = table ? ttot / kChunk + B + 1 : (int64_t)B * nps64;
    if (nch64 * H > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    const int nch = (int)nch64;

    const size_t segs_b = table ? (size_t)nch * sizeof(SegEntry) : 0;
    const size_t seqs_b = table ? ((size_t)B * sizeof(SeqEntry) + 255) / 256 * 256 : 0;
    // Per chunk and head: W (64 x 128 bf16) and U (64 x 128 fp32), then
    // new_v (64 x 128 bf16) for the output kernel.
    const size_t tiles_b = (size_t)nch * H * kChunk * 128 * (sizeof(uint16_t) + sizeof(float));
    const size_t nv_b = (size_t)nch * H * kChunk * 128 * sizeof(uint16_t);
    const size_t ws_b = segs_b + seqs_b + tiles_b + nv_b;
    char *ws = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&ws), ws_b, st);
    if (e != hipSuccess) return SGLA_ERR_HIP;

    GdnParams p{};
    p.c.q = q;
    p.c.k = k;
    p.c.v = v;
    p.c.g = g;
    p.c.s0 = initial_state;
    p.c.out = out;
    p.c.sfin = final_state;
    p.c.segs = table ? reinterpret_cast<SegEntry *>(ws) : nullptr;
    p.c.seqs = table ? reinterpret_cast<SeqEntry *>(ws + segs_b) : nullptr;
    p.c.H = H;
    p.c.nseg_max = nch;
    p.c.N = B;
    p.c.scale = scale;
    p.c.T = T;
    p.c.seg_len = kChunk;
    p.c.nps = (int)nps64;
    p.beta = beta;
    p.tiles = ws + segs_b + seqs_b;
    p.nvimg = ws + segs_b + seqs_b + tiles_b;
    if (table)
        e = launch_plan(cu_seqlens, B, T, kChunk, nch, reinterpret_cast<SegEntry *>(ws),
                        reinterpret_cast<SeqEntry *>(ws + segs_b), st);
    if (e == hipSuccess) e = launch_gdn_chunk(p, st);
    const hipError_t ef = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = ef;
    return hip_status(e);
}

sgla_status sgla_gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, float *state,
                                    const int32_t *state_indices, void *out, int N, int H, int Dk,
                                    int Dv, float scale, sgla_dtype dtype, void *stream) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    if (!head_size_ok(Dk) || !head_size_ok(Dv)) return SGLA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > ((int64_t)1 << 31) - 1) return SGLA_ERR_INVALID_ARG;
    if (N == 0) return SGLA_OK;
    if (!q || !k || !v || !g || !beta || !state || !out) return SGLA_ERR_INVALID_ARG;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g, 4) ||
        misaligned(beta, 4) || misaligned(state) || misaligned(out) ||
        misaligned(state_indices, 4))
        return SGLA_ERR_INVALID_ARG;
    return hip_status(launch_gdn_step(q, k, v, g, beta, state, state_indices, out, N, H, Dk, Dv,
                                      scale, dtype == SGLA_BF16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
