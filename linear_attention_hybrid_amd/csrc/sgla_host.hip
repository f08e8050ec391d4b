// Host side of the libsgla C ABI: argument checks, planning, launches.
#include <stdlib.h>
#include <string.h>

#include <mutex>

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
// Below this many (sub-segment, head) units the state pass runs over value
// halves: the compute units of one MI355X.
constexpr int64_t kStateHalvesUnits = 256;

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
// 1024 tokens (16 chunks) and whole chunks. pre_units = (segment, head) pairs
// whose state is needed when each output segment is one sub-segment.
// Measured on the 8192-token call (1024-token output segments): one
// sub-segment each, 104.1 us flushed, against 111.2 us with two of 512
// tokens and 140.0 us with four (shorter workgroups spend more of their time
// waiting for their first chunk, and the output workgroups combine twice the
// states); on the 65,536-token call two 4096-token sub-segments stay best
// (707.6 us flushed, against 737.7 us with one and 755.5 us with four).
int choose_rsub(int out_len, int64_t pre_units) {
    const char *env = getenv("SGLA_RSUB");
    if (env) {
        long v = strtol(env, nullptr, 10);
        if (v >= 1 && v <= out_len / kChunk && (out_len / kChunk) % v == 0) return (int)v;
    }
    int r = 1;
    while (out_len / (2 * r) >= 1024 && (out_len / kChunk) % (2 * r) == 0 && pre_units * r < 384) r *= 2;
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

// The plan of one chunked Simple GLA call: which kernels run, how sequences
// are cut into segments, and where the tables and states sit in the caller's
// workspace (a 256-byte header first: word 0 receives the cu_seqlens check
// when SGLA_VALIDATE is set). Computed the same way for the workspace-size
// query and for the call.
struct ChunkPlan {
    bool halves = false;   // value-half output kernel (bf16, 128-wide heads, no prologue)
    bool mfma = false;     // one-level kernels on the matrix cores (else the vector ALUs)
    bool table = false;    // segment tables built on the device from cu_seqlens
    bool split = false;    // state pass and scan (some sequence spans several segments)
    int seg_len = 0;       // one-level segments, or the state pass's sub-segments
    int64_t nps = 1;       // segments per sequence without a table
    int64_t nseg = 0;      // table rows (segments) of the one-level or state pass
    int rsub = 1;          // sub-segments per output segment (value halves)
    bool state_halves = false;  // state pass over value-column halves (see below)
    int oseg_len = 0;      // value-half output segments
    int64_t onps = 1;
    int64_t onseg = 0;
    size_t off_osegs = 0, off_oseqs = 0, off_segs = 0, off_seqs = 0, off_gam = 0, off_buf = 0;
    size_t bytes = 0;      // workspace bytes (0: none)
};

sgla_status make_plan(int B, int T, int H, int Dk, int Dv, sgla_dtype dtype, bool varlen, bool pro,
                      bool split_ok, ChunkPlan &pl);
sgla_status chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, void *out, float *final_state,
                      const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv, float scale,
                      sgla_dtype dtype, void *stream, const ProArgs *pro, void *workspace,
                      size_t workspace_bytes);

}  // namespace

extern "C" {

const char *sgla_status_string(sgla_status s) {
    switch (s) {
        case SGLA_OK: return "SGLA_OK";
        case SGLA_ERR_INVALID_ARG: return "SGLA_ERR_INVALID_ARG";
        case SGLA_ERR_UNSUPPORTED: return "SGLA_ERR_UNSUPPORTED";
        case SGLA_ERR_HIP: return "SGLA_ERR_HIP";
        case SGLA_ERR_WORKSPACE: return "SGLA_ERR_WORKSPACE";
    }
    return "SGLA_ERR_UNKNOWN";
}

int sgla_version(void) { return kVersion; }

sgla_status sgla_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                           const float *initial_state, void *out, float *final_state,
                           const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                           float scale, sgla_dtype dtype, void *stream) {
    return chunk_fwd(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H, Dk, Dv,
                     scale, dtype, stream, nullptr, nullptr, 0);
}

sgla_status sgla_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, sgla_dtype dtype,
                                          int varlen, int prologue, size_t *bytes) {
    if (!bytes) return SGLA_ERR_INVALID_ARG;
    *bytes = 0;
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    if (!head_size_ok(Dk) || !head_size_ok(Dv) || H > kMaxHeads) return SGLA_ERR_UNSUPPORTED;
    if (prologue && (dtype != SGLA_BF16 || Dk != 128 || Dv != 128)) return SGLA_ERR_UNSUPPORTED;
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    if ((int64_t)B * H > (int64_t)1 << 30) return SGLA_ERR_INVALID_ARG;
    if (B == 0) return SGLA_OK;
    ChunkPlan pl;
    const sgla_status st = make_plan(B, T, H, Dk, Dv, dtype, varlen != 0, prologue != 0, true, pl);
    if (st == SGLA_OK) *bytes = pl.bytes;
    return st;
}

sgla_status sgla_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *initial_state, void *out, float *final_state,
                              const int64_t *cu_seqlens, const float *q_weight,
                              const float *k_weight, const int32_t *pos_offset, float theta,
                              float eps, int B, int T, int H, int Dk, int Dv, float scale,
                              sgla_dtype dtype, void *workspace, size_t workspace_bytes,
                              void *stream) {
    const ProArgs pro{q_weight, k_weight, pos_offset, theta, eps};
    return chunk_fwd(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H, Dk, Dv,
                     scale, dtype, stream, q_weight ? &pro : nullptr, workspace, workspace_bytes);
}

sgla_status sgla_qk_norm_rope(const void *x, const float *weight, const int32_t *pos_offset,
                              void *out, int B, int T, int H, int Dk, float theta, float eps,
                              sgla_dtype dtype, void *stream) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 1 || Dk < 1) return SGLA_ERR_INVALID_ARG;
    if (dtype != SGLA_BF16 || Dk != 128 || H > kMaxHeads) return SGLA_ERR_UNSUPPORTED;
    const ProArgs pro{weight, weight, pos_offset, theta, eps};
    const sgla_status ps = check_prologue(pro);
    if (ps != SGLA_OK) return ps;
    const int64_t units = (int64_t)B * ((T + 63) / 64) * H;
    if (units > ((int64_t)1 << 31) - 1) return SGLA_ERR_UNSUPPORTED;
    if (units == 0) return SGLA_OK;
    if (!x || !out || misaligned(x) || misaligned(out)) return SGLA_ERR_INVALID_ARG;
    return hip_status(launch_qk_norm_rope(x, weight, pos_offset, out, B, T, H, theta, eps,
                                          static_cast<hipStream_t>(stream)));
}

sgla_status sgla_validate_cu_seqlens(const int64_t *cu_seqlens, int B, int T, int32_t *status,
                                     void *stream) {
    if (B < 0 || T < 0 || !status || !cu_seqlens) return SGLA_ERR_INVALID_ARG;
    if (misaligned(cu_seqlens, 8) || misaligned(status, 4)) return SGLA_ERR_INVALID_ARG;
    return hip_status(launch_validate_cu(cu_seqlens, B, T, status, static_cast<hipStream_t>(stream)));
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
                     scale, dtype, stream, &pro, nullptr, 0);
}

}  // extern "C"

namespace {

constexpr size_t kWsHeader = 256;

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// split_ok: a workspace may be used. Without one, every sequence is one
// segment (one workgroup per sequence and head, or per sequence, head and
// value half), which needs no tables and no states.
sgla_status make_plan(int B, int T, int H, int Dk, int Dv, sgla_dtype dtype, bool varlen, bool pro,
                      bool split_ok, ChunkPlan &pl) {
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    const bool bf16 = dtype == SGLA_BF16;
    // bf16 with 128-wide heads and no prologue: equal-length batches run on
    // the value-half kernels (less state traffic; as fast on 8K-token
    // sequences and faster on long ones). Packed sequences of mixed lengths
    // stay on the one-level kernels, whose shorter segments balance better:
    // there the per-chunk work bounds the call, and the value halves repeat
    // the scores. Without a workspace (one segment per sequence) the value
    // halves give twice the workgroups. SGLA_VALUE_HALVES / SGLA_ONE_LEVEL
    // force either path.
    const bool mfma_ok = bf16 && Dk == 128 && Dv == 128 && !getenv("SGLA_FORCE_VALU");
    const bool want_halves = getenv("SGLA_ONE_LEVEL") ? false
                             : getenv("SGLA_VALUE_HALVES") ? true
                             : !varlen || !split_ok;
    pl.halves = mfma_ok && !pro && want_halves;
    pl.mfma = bf16 && Dk == 128 && Dv == 128 && (pro || !getenv("SGLA_FORCE_VALU"));
    const int whole = T <= 0 ? kChunk : (int)(((int64_t)T + kChunk - 1) / kChunk * kChunk);
    size_t off = kWsHeader;
    if (pl.halves) {
        pl.oseg_len = split_ok ? choose_out_len(ttot, H) : whole;
        pl.onps = T == 0 ? 1 : ((int64_t)T + pl.oseg_len - 1) / pl.oseg_len;
        pl.table = varlen && split_ok;
        pl.onseg = varlen ? (pl.table ? ttot / pl.oseg_len + B + 1 : B) : (int64_t)B * pl.onps;
        if (pl.onseg * H * 2 > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
        pl.split = pl.table || pl.onps > 1;
        const int64_t pre_units = varlen ? (ttot / pl.oseg_len) * H : (pl.onps - 1) * B * H;
        pl.rsub = pl.split ? choose_rsub(pl.oseg_len, pre_units) : 1;
        // The state pass over value-column halves, when one workgroup per
        // (sub-segment, head) would leave compute units idle. Measured: on
        // the 8192-token call (224 units) 108.3 against 109.5 us flushed;
        // on the 65,536-token call (448 units) 756 against 712 us and on
        // the 524,288-token varlen call 6.19 against 5.94 ms, so not there.
        pl.state_halves = pl.split && pre_units * pl.rsub < kStateHalvesUnits;
        pl.seg_len = pl.oseg_len / pl.rsub;
        pl.nps = T == 0 ? 1 : ((int64_t)T + pl.seg_len - 1) / pl.seg_len;
        pl.nseg = !pl.split ? 0 : pl.table ? ttot / pl.seg_len + B + 1 : (int64_t)B * pl.nps;
        if (pl.nseg * H > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
        if (pl.table) {
            pl.off_osegs = off; off += round256((size_t)pl.onseg * sizeof(SegEntry));
            pl.off_oseqs = off; off += round256((size_t)B * sizeof(SeqEntry));
        }
    } else {
        pl.seg_len = split_ok ? choose_seg_len(ttot, B, H) : whole;
        pl.nps = T == 0 ? 1 : ((int64_t)T + pl.seg_len - 1) / pl.seg_len;
        pl.table = varlen && split_ok;
        pl.nseg = varlen ? (pl.table ? ttot / pl.seg_len + B + 1 : B) : (int64_t)B * pl.nps;
        // The vector-ALU kernels run one workgroup per 32 value columns of
        // each (segment, head); every grid must stay below 2^31.
        if (pl.nseg * H * ((Dv + 31) / 32) > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
        pl.split = pl.table || pl.nps > 1;
    }
    if (pl.table) {
        pl.off_segs = off; off += round256((size_t)pl.nseg * sizeof(SegEntry));
        pl.off_seqs = off; off += round256((size_t)B * sizeof(SeqEntry));
    }
    if (pl.split) {
        pl.off_gam = off; off += round256((size_t)pl.nseg * H * sizeof(float));
        pl.off_buf = off; off += (size_t)pl.nseg * H * Dk * Dv * sizeof(float);
    }
    pl.bytes = (pl.table || pl.split) ? off : 0;
    return SGLA_OK;
}

sgla_status check_chunk_args(const void *q, const void *k, const void *v, const float *g,
                             const float *initial_state, const void *out, const float *final_state,
                             const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                             sgla_dtype dtype, const ProArgs *pro) {
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
    return SGLA_OK;
}

sgla_status chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                      const float *initial_state, void *out, float *final_state,
                      const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv, float scale,
                      sgla_dtype dtype, void *stream, const ProArgs *pro, void *workspace,
                      size_t workspace_bytes) {
    sgla_status stt = check_chunk_args(q, k, v, g, initial_state, out, final_state, cu_seqlens, B,
                                       T, H, Dk, Dv, dtype, pro);
    if (stt != SGLA_OK) return stt;
    if (misaligned(workspace, 256)) return SGLA_ERR_INVALID_ARG;
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (B == 0) return SGLA_OK;
    if (ttot == 0 && !final_state) return SGLA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);

    ChunkPlan pl;
    stt = make_plan(B, T, H, Dk, Dv, dtype, cu_seqlens != nullptr, pro != nullptr,
                    workspace != nullptr, pl);
    if (stt != SGLA_OK) return stt;
    if (pl.bytes > workspace_bytes) return SGLA_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    auto at = [&](size_t off) -> char * { return ws ? ws + off : nullptr; };

    ChunkParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.s0 = initial_state;
    p.out = out;
    p.sfin = final_state;
    p.cu = pl.table ? nullptr : cu_seqlens;
    p.segs = pl.table ? reinterpret_cast<SegEntry *>(at(pl.off_segs)) : nullptr;
    p.seqs = pl.table ? reinterpret_cast<SeqEntry *>(at(pl.off_seqs)) : nullptr;
    p.gam = pl.split ? reinterpret_cast<float *>(at(pl.off_gam)) : nullptr;
    p.buf = pl.split ? reinterpret_cast<float *>(at(pl.off_buf)) : nullptr;
    p.H = H;
    p.nseg_max = (int)pl.nseg;
    p.N = B;
    p.scale = scale;
    p.T = T;
    p.seg_len = pl.seg_len;
    p.nps = (int)pl.nps;
    p.qw = pro ? pro->qw : nullptr;
    p.kw = pro ? pro->kw : nullptr;
    p.pos_off = pro ? pro->pos : nullptr;
    p.theta = pro ? pro->theta : 0.f;
    p.eps = pro ? pro->eps : 0.f;
    p.rsub = pl.rsub;
    p.state_halves = pl.state_halves ? 1 : 0;
    const bool bf16 = dtype == SGLA_BF16;

    hipError_t e = hipSuccess;
    if (cu_seqlens && ws && getenv("SGLA_VALIDATE"))
        e = launch_validate_cu(cu_seqlens, B, T, reinterpret_cast<int32_t *>(ws), st);
    if (pl.halves) {
        HalvesParams hp{};
        hp.c = p;
        hp.osegs = pl.table ? reinterpret_cast<SegEntry *>(at(pl.off_osegs)) : nullptr;
        hp.onseg_max = (int)pl.onseg;
        hp.onps = (int)pl.onps;
        hp.oseg_len = pl.oseg_len;
        if (e == hipSuccess && pl.table) {
            e = launch_plan(cu_seqlens, B, T, pl.oseg_len, (int)pl.onseg,
                            reinterpret_cast<SegEntry *>(at(pl.off_osegs)),
                            reinterpret_cast<SeqEntry *>(at(pl.off_oseqs)), st);
            if (e == hipSuccess)
                e = launch_plan(cu_seqlens, B, T, pl.seg_len, (int)pl.nseg,
                                reinterpret_cast<SegEntry *>(at(pl.off_segs)),
                                reinterpret_cast<SeqEntry *>(at(pl.off_seqs)), st);
        }
        // The output kernel combines the sub-segment states itself (no scan).
        if (e == hipSuccess && pl.split) e = launch_chunk_mfma(p, /*phase_state=*/true, st);
        if (e == hipSuccess) e = launch_chunk_halves(hp, st);
        return hip_status(e);
    }
    auto phase = [&](bool state_phase) {
        return pl.mfma ? launch_chunk_mfma(p, state_phase, st)
                       : launch_chunk_valu(p, bf16, Dk, Dv, state_phase, st);
    };
    if (e == hipSuccess && pl.table)
        e = launch_plan(cu_seqlens, B, T, pl.seg_len, (int)pl.nseg,
                        reinterpret_cast<SegEntry *>(at(pl.off_segs)),
                        reinterpret_cast<SeqEntry *>(at(pl.off_seqs)), st);
    if (e == hipSuccess && pl.split) e = phase(/*state_phase=*/true);
    if (e == hipSuccess && pl.split) e = launch_scan(p, Dk, Dv, st);
    if (e == hipSuccess) e = phase(/*state_phase=*/false);
    return hip_status(e);
}

// Scratch space of sgla_chunk_fwd_noalloc: one array per GPU, in the code
// object's device memory, held until the process ends. Host code must not use
// the array's name as an address (it names a host-side stand-in): the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device,
// with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void *scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

hipError_t scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(scratch_once[dev], [dev] {
        void *p = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        scratch_ptr[dev] = p;
    });
    if (scratch_err[dev] != hipSuccess) return scratch_err[dev];
    *out = scratch_ptr[dev];
    return hipSuccess;
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

sgla_status sgla_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                                   const float *initial_state, void *out, float *final_state,
                                   const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                                   float scale, sgla_dtype dtype, void *stream) {
    const sgla_status st = check_chunk_args(q, k, v, g, initial_state, out, final_state,
                                            cu_seqlens, B, T, H, Dk, Dv, dtype, nullptr);
    if (st != SGLA_OK) return st;
    void *ws = nullptr;
    if (scratch_of_current_device(&ws) != hipSuccess) return SGLA_ERR_HIP;
    return chunk_fwd(q, k, v, g, initial_state, out, final_state, cu_seqlens, B, T, H, Dk, Dv,
                     scale, dtype, stream, nullptr, ws, kScratchBytes);
}

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

}  // extern "C"

namespace {

// Workspace layout of the chunked gated delta rule: a 256-byte header, the
// chunk tables (with cu_seqlens), then per (chunk, head) the W/U tile and the
// new_v image.
struct GdnPlan {
    bool table = false;
    int64_t nps = 1, nch = 0;
    size_t off_segs = 0, off_seqs = 0, off_tiles = 0, off_nv = 0, bytes = 0;
};

sgla_status gdn_plan(int B, int T, int H, bool varlen, GdnPlan &pl) {
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    pl.table = varlen;
    pl.nps = T == 0 ? 1 : ((int64_t)T + kChunk - 1) / kChunk;
    pl.nch = varlen ? ttot / kChunk + B + 1 : (int64_t)B * pl.nps;
    if (pl.nch * H > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    size_t off = kWsHeader;
    if (pl.table) {
        pl.off_segs = off; off += round256((size_t)pl.nch * sizeof(SegEntry));
        pl.off_seqs = off; off += round256((size_t)B * sizeof(SeqEntry));
    }
    // Per chunk and head: W (64 x 128 bf16) and U (64 x 128 fp32), then
    // new_v (64 x 128 bf16) for the output kernel.
    pl.off_tiles = off; off += (size_t)pl.nch * H * kChunk * 128 * (sizeof(uint16_t) + sizeof(float));
    pl.off_nv = off; off += (size_t)pl.nch * H * kChunk * 128 * sizeof(uint16_t);
    pl.bytes = off;
    return SGLA_OK;
}

sgla_status check_gdn_args(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *initial_state, const void *out,
                           const float *final_state, const int64_t *cu_seqlens, int B, int T,
                           int H, int Dk, int Dv, sgla_dtype dtype) {
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
    return SGLA_OK;
}

sgla_status gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, void *out,
                          float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                          int Dk, int Dv, float scale, sgla_dtype dtype, void *workspace,
                          size_t workspace_bytes, void *stream) {
    sgla_status stt = check_gdn_args(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                                     B, T, H, Dk, Dv, dtype);
    if (stt != SGLA_OK) return stt;
    if (misaligned(workspace, 256)) return SGLA_ERR_INVALID_ARG;
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (B == 0) return SGLA_OK;
    if (ttot == 0 && !final_state) return SGLA_OK;
    GdnPlan pl;
    stt = gdn_plan(B, T, H, cu_seqlens != nullptr, pl);
    if (stt != SGLA_OK) return stt;
    if (!workspace || pl.bytes > workspace_bytes) return SGLA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    GdnParams p{};
    p.c.q = q;
    p.c.k = k;
    p.c.v = v;
    p.c.g = g;
    p.c.s0 = initial_state;
    p.c.out = out;
    p.c.sfin = final_state;
    p.c.segs = pl.table ? reinterpret_cast<SegEntry *>(ws + pl.off_segs) : nullptr;
    p.c.seqs = pl.table ? reinterpret_cast<SeqEntry *>(ws + pl.off_seqs) : nullptr;
    p.c.H = H;
    p.c.nseg_max = (int)pl.nch;
    p.c.N = B;
    p.c.scale = scale;
    p.c.T = T;
    p.c.seg_len = kChunk;
    p.c.nps = (int)pl.nps;
    p.c.rsub = 1;
    p.beta = beta;
    p.tiles = ws + pl.off_tiles;
    p.nvimg = ws + pl.off_nv;
    hipError_t e = hipSuccess;
    if (cu_seqlens && getenv("SGLA_VALIDATE"))
        e = launch_validate_cu(cu_seqlens, B, T, reinterpret_cast<int32_t *>(ws), st);
    if (e == hipSuccess && pl.table)
        e = launch_plan(cu_seqlens, B, T, kChunk, (int)pl.nch,
                        reinterpret_cast<SegEntry *>(ws + pl.off_segs),
                        reinterpret_cast<SeqEntry *>(ws + pl.off_seqs), st);
    if (e == hipSuccess) e = launch_gdn_chunk(p, st);
    return hip_status(e);
}

// One delta-rule decode token per row (GDN: g [N, H]; KDA: g [N, H, Dk]).
sgla_status delta_step(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, float *state, const int32_t *state_indices, void *out,
                       int N, int H, int Dk, int Dv, float scale, sgla_dtype dtype, bool kda,
                       void *stream) {
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
                                      scale, dtype == SGLA_BF16, kda,
                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

sgla_status sgla_gdn_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv,
                                              sgla_dtype dtype, int varlen, size_t *bytes) {
    if (!bytes) return SGLA_ERR_INVALID_ARG;
    *bytes = 0;
    sgla_status st = check_gdn_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, B, 0, H, Dk, Dv, dtype);
    if (st != SGLA_OK) return st;
    if (T < 0) return SGLA_ERR_INVALID_ARG;
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    if (B == 0) return SGLA_OK;
    GdnPlan pl;
    st = gdn_plan(B, T, H, varlen != 0, pl);
    if (st == SGLA_OK) *bytes = pl.bytes;
    return st;
}

sgla_status sgla_gdn_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state, void *out,
                                  float *final_state, const int64_t *cu_seqlens, int B, int T,
                                  int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, B, T, H,
                         Dk, Dv, scale, dtype, workspace, workspace_bytes, stream);
}

sgla_status sgla_gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, void *out,
                               float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                               int Dk, int Dv, float scale, sgla_dtype dtype, void *stream) {
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, B, T, H,
                         Dk, Dv, scale, dtype, nullptr, 0, stream);
}

sgla_status sgla_gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, float *state,
                                    const int32_t *state_indices, void *out, int N, int H, int Dk,
                                    int Dv, float scale, sgla_dtype dtype, void *stream) {
    return delta_step(q, k, v, g, beta, state, state_indices, out, N, H, Dk, Dv, scale, dtype,
                      false, stream);
}

sgla_status sgla_kda_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, float *state,
                                    const int32_t *state_indices, void *out, int N, int H, int Dk,
                                    int Dv, float scale, sgla_dtype dtype, void *stream) {
    return delta_step(q, k, v, g, beta, state, state_indices, out, N, H, Dk, Dv, scale, dtype,
                      true, stream);
}

}  // extern "C"

namespace {

// Workspace layout of the chunked KDA: a 256-byte header, the chunk tables
// (with cu_seqlens), then per (chunk, head) the prep tile, new_v and the
// chunk's start state.
struct KdaPlan {
    bool table = false;
    int64_t nps = 1, nch = 0;
    size_t off_segs = 0, off_seqs = 0, off_tiles = 0, off_nv = 0, off_sin = 0, bytes = 0;
};

sgla_status kda_plan(int B, int T, int H, int Dk, int Dv, bool varlen, KdaPlan &pl) {
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    pl.table = varlen;
    pl.nps = T == 0 ? 1 : ((int64_t)T + kChunk - 1) / kChunk;
    pl.nch = varlen ? ttot / kChunk + B + 1 : (int64_t)B * pl.nps;
    if (pl.nch * H > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    size_t off = kWsHeader;
    if (pl.table) {
        pl.off_segs = off; off += round256((size_t)pl.nch * sizeof(SegEntry));
        pl.off_seqs = off; off += round256((size_t)B * sizeof(SeqEntry));
    }
    const size_t units = (size_t)pl.nch * H;
    const size_t tile = (size_t)(2 * kChunk * Dk + kChunk * Dv + Dk) * sizeof(float);
    pl.off_tiles = off; off += round256(units * tile);
    pl.off_nv = off; off += round256(units * kChunk * Dv * sizeof(float));
    pl.off_sin = off; off += round256(units * Dk * Dv * sizeof(float));
    pl.bytes = off;
    return SGLA_OK;
}

sgla_status check_kda_args(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *initial_state, const void *out,
                           const float *final_state, const int64_t *cu_seqlens, int B, int T,
                           int H, int Dk, int Dv, sgla_dtype dtype) {
    if (dtype != SGLA_F32 && dtype != SGLA_BF16) return SGLA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return SGLA_ERR_INVALID_ARG;
    if (!head_size_ok(Dk) || !head_size_ok(Dv) || H > kMaxHeads) return SGLA_ERR_UNSUPPORTED;
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    // The chain kernel runs Dv / 16 workgroups per (sequence, head).
    if ((int64_t)B * H * (Dv / 16) > ((int64_t)1 << 31) - 64) return SGLA_ERR_UNSUPPORTED;
    if (ttot > 0 && (!q || !k || !v || !g || !beta || !out)) return SGLA_ERR_INVALID_ARG;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) ||
        misaligned(beta, 4) || misaligned(out) || misaligned(initial_state) ||
        misaligned(final_state) || misaligned(cu_seqlens, 8))
        return SGLA_ERR_INVALID_ARG;
    return SGLA_OK;
}

sgla_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, void *out,
                          float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                          int Dk, int Dv, float scale, sgla_dtype dtype, void *workspace,
                          size_t workspace_bytes, void *stream) {
    sgla_status stt = check_kda_args(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens,
                                     B, T, H, Dk, Dv, dtype);
    if (stt != SGLA_OK) return stt;
    if (misaligned(workspace, 256)) return SGLA_ERR_INVALID_ARG;
    const int64_t ttot = cu_seqlens ? (int64_t)T : (int64_t)B * T;
    if (B == 0) return SGLA_OK;
    if (ttot == 0 && !final_state) return SGLA_OK;
    KdaPlan pl;
    stt = kda_plan(B, T, H, Dk, Dv, cu_seqlens != nullptr, pl);
    if (stt != SGLA_OK) return stt;
    if (!workspace || pl.bytes > workspace_bytes) return SGLA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    KdaParams p{};
    p.c.q = q;
    p.c.k = k;
    p.c.v = v;
    p.c.g = g;
    p.c.s0 = initial_state;
    p.c.out = out;
    p.c.sfin = final_state;
    p.c.segs = pl.table ? reinterpret_cast<SegEntry *>(ws + pl.off_segs) : nullptr;
    p.c.seqs = pl.table ? reinterpret_cast<SeqEntry *>(ws + pl.off_seqs) : nullptr;
    p.c.H = H;
    p.c.nseg_max = (int)pl.nch;
    p.c.N = B;
    p.c.scale = scale;
    p.c.T = T;
    p.c.seg_len = kChunk;
    p.c.nps = (int)pl.nps;
    p.c.rsub = 1;
    p.beta = beta;
    p.tiles = reinterpret_cast<float *>(ws + pl.off_tiles);
    p.nv = reinterpret_cast<float *>(ws + pl.off_nv);
    p.sin = reinterpret_cast<float *>(ws + pl.off_sin);
    p.dk = Dk;
    p.dv = Dv;
    hipError_t e = hipSuccess;
    if (cu_seqlens && getenv("SGLA_VALIDATE"))
        e = launch_validate_cu(cu_seqlens, B, T, reinterpret_cast<int32_t *>(ws), st);
    if (e == hipSuccess && pl.table)
        e = launch_plan(cu_seqlens, B, T, kChunk, (int)pl.nch,
                        reinterpret_cast<SegEntry *>(ws + pl.off_segs),
                        reinterpret_cast<SeqEntry *>(ws + pl.off_seqs), st);
    if (e == hipSuccess) e = launch_kda_chunk(p, dtype == SGLA_BF16, st);
    return hip_status(e);
}

}  // namespace

extern "C" {

sgla_status sgla_kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv,
                                              sgla_dtype dtype, int varlen, size_t *bytes) {
    if (!bytes) return SGLA_ERR_INVALID_ARG;
    *bytes = 0;
    sgla_status st = check_kda_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, B, 0, H, Dk, Dv, dtype);
    if (st != SGLA_OK) return st;
    if (T < 0) return SGLA_ERR_INVALID_ARG;
    const int64_t ttot = varlen ? (int64_t)T : (int64_t)B * T;
    if (ttot > ((int64_t)1 << 62) / ((int64_t)H * 128)) return SGLA_ERR_INVALID_ARG;
    if (B == 0) return SGLA_OK;
    KdaPlan pl;
    st = kda_plan(B, T, H, Dk, Dv, varlen != 0, pl);
    if (st == SGLA_OK) *bytes = pl.bytes;
    return st;
}

sgla_status sgla_kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state, void *out,
                                  float *final_state, const int64_t *cu_seqlens, int B, int T,
                                  int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    return kda_chunk_fwd(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, B, T, H,
                         Dk, Dv, scale, dtype, workspace, workspace_bytes, stream);
}

sgla_status sgla_kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, void *out,
                               float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                               int Dk, int Dv, float scale, sgla_dtype dtype, void *stream) {
    return kda_chunk_fwd(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, B, T, H,
                         Dk, Dv, scale, dtype, nullptr, 0, stream);
}

}  // extern "C"
