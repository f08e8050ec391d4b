// Chunked Simple GLA on the matrix cores: bf16 operands, fp32 accumulation,
// Dk = Dv = 128, chunks of 64 tokens.
//
// Per chunk with inclusive cumulative gate sums G (page "Formulas and code for
// adapting inference to GDN/KDA linear modules", section 1.2, reduced to Simple
// GLA: no delta-rule terms, new_v = v; the diagonal is included because the
// query reads the state after the token's own update, blueprint page, section
// "B2 lightning-attn (Simple GLA)"):
//
//   A^T = K Q^T, then A[i][j] = scale * exp(G_i - G_j) * (q_i . k_j) for j <= i, else 0
//   O^T = S^T Q^T (rows scaled by scale * exp(G_i)) + V^T A^T
//   S   = exp(G_last) * S + (K * exp(G_last - G))^T V
//
// Everything is written in transposed form so that each MFMA result is
// already in the register layout the next MFMA consumes:
//   * the fp32 state S lives in the accumulators of the state update
//     (32x32 tiles: lane l holds S[dk rows 8(v/4)+4(l/32)+v%4][dv column l%32]);
//     converted in registers to a bf16 pair hi + lo it is directly the A
//     operand of S^T Q^T (two MFMAs), with Q read in the matching order of
//     its dk rows. The pair keeps about 16 bits of the state: one bf16
//     rounding of a large, slowly decaying state would cost the outputs 2^-9
//     of their size;
//   * A^T = K Q^T leaves each lane one query column i and 16 key rows j, i.e.
//     4 consecutive j per group, written to LDS as A[i][j] with 8-byte stores,
//     and read back as the B operand of V^T A^T;
//   * O^T leaves each lane one token column i and 4 consecutive value rows per
//     group, written to LDS as O[i][dv] rows and stored to HBM 16 B per lane.
//
// A workgroup is 4 waves; wave w owns value columns [32w, 32w+32) of the state
// and of the output. Per chunk the workgroup streams q, k, v (16 KiB each) and
// g from HBM with 16-byte buffer loads, one chunk ahead of the compute
// (registers); the buffer range check zeroes the rows past the end of a ragged
// chunk and drops their output stores. It stages the tiles in LDS: Q and K row-major with 16-byte chunks XOR-swizzled by
// row, K*exp(G_last-G) and V transposed (token-contiguous) with a swizzle that
// keeps both the transposing writes and the MFMA operand reads spread over the
// banks. LDS: 72 KiB for the output phase, so two workgroups fit on a CU.
#include "mfma_tile.h"

namespace sgla {

namespace {

constexpr int D = 128;
constexpr int NT = 256;
// LDS map, bytes.
constexpr int OFF_Q = 0;          // Q rows [64][256 B], chunk-swizzled
constexpr int OFF_K = 16384;      // K rows [64][256 B]; later the O staging rows
constexpr int OFF_KT = 32768;     // (K*exp(G_last-G))^T [128 dk][128 B]
constexpr int OFF_VT = 49152;     // V^T [128 dv][128 B]
constexpr int OFF_A = 65536;      // A[64 i][128 B]
constexpr int OFF_G = 73728;      // G[64] fp32
constexpr int LDS_OUT = OFF_G + 256;
constexpr int LDS_STATE = 32768;  // KT and VT only (state phase, placed at 0)
// q/k prologue tables, after the kernel's own LDS: RMSNorm weights of q and
// k (2 x 128 fp32), RoPE turns per position per frequency (64 fp64), cos and sin of one position's and of 32 positions' turn per
// frequency (2 x 64 x 2 fp32), and each wave's turns of its four rows of the
// current chunk (4 x 4 x 64 fp32).
constexpr int PRO_W = 0;
constexpr int PRO_OM = 1024;
constexpr int PRO_ROT = 1792;
constexpr int PRO_ROT32 = 2304;
constexpr int PRO_BASE = 2816;   // per wave: turns of its 4 rows x 64 frequencies (4 x 1 KiB)
constexpr int PRO_BYTES = PRO_BASE + 4 * 1024;
// Two workgroups per CU (amdgpu_waves_per_eu(2), four waves each).
static_assert(2 * (LDS_OUT + PRO_BYTES) <= kLdsPerCU, "two output workgroups must fit one CU's LDS");
static_assert(2 * (LDS_STATE + PRO_BYTES) <= kLdsPerCU, "two state workgroups must fit one CU's LDS");

// The prologue of one 16-byte piece (8 consecutive dims 8c .. 8c+7 of a
// 128-dim row, c = lane & 15) held by each of the 16 lanes of a DPP row:
// RMSNorm over the row (sum of squares across the 16 lanes), weight, bf16;
// then RoPE against the partner dims (c ^ 8, the other half of the row), bf16.
// cs/sn are the cos and sin of each dim's angle, the sine already negated in
// the lower half (c < 8), where the partner enters with a minus sign. `ok`
// false (a row past the end of the chunk) gives zeros.
__device__ __forceinline__ u32x4 qk_prologue_piece(u32x4 raw, const char *lds, int w_off,
                                                   const float cs[8], const float sn[8], bool ok,
                                                   float eps) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = lo_bf16(raw[j]);
        x[2 * j + 1] = hi_bf16(raw[j]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = row16_sum(ss);
    const float rs = ok ? rsqrtf(ss * (1.f / D) + eps) : 0.f;
    const float4 w0 = lds_ld<float4>(lds, w_off);
    const float4 w1 = lds_ld<float4>(lds, w_off + 16);
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = round_bf16(x[e] * rs * w[e]);
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 2 * j + h;
            const float t = row16_swap8(y[e]) * sn[e];
            o[h] = fmaf(y[e], cs[e], t);
        }
        r[j] = pack_f32(o[0], o[1]);
    }
    return r;
}

// The prologue tables in LDS at `base` (PRO_BYTES): the two RMSNorm weight
// vectors (q's skipped when qw is null), the turns per position of each
// frequency (fp64), and the cos and sin of one position's and of 32
// positions' turn per frequency. Callers synchronise before reading them.
__device__ __forceinline__ void prologue_tables(char *lds, int base, const float *qw,
                                                const float *kw, float theta, int tid) {
    if (tid < D) {
        if (qw) lds_st(lds, base + PRO_W + 4 * tid, qw[tid]);
        lds_st(lds, base + PRO_W + 512 + 4 * tid, kw[tid]);
    }
    if (tid < 64) {
        const double om = rope_turns_per_pos(tid, D, theta);
        lds_st(lds, base + PRO_OM + 8 * tid, om);
        const double t = 6.283185307179586477 * (om - rint(om));
        lds_st(lds, base + PRO_ROT + 8 * tid, make_float2((float)cos(t), (float)sin(t)));
        const double t32 = 6.283185307179586477 * (32.0 * om - rint(32.0 * om));
        lds_st(lds, base + PRO_ROT32 + 8 * tid, make_float2((float)cos(t32), (float)sin(t32)));
    }
}

// The prologue of one 64-token chunk on the registers of one thread: its
// 16-byte pieces (dims 8c .. 8c+7, c = tid & 15) of rows 2 prb + 32 it + rr
// (prb = (tid >> 4) & 15) of k, and of q when Q. pos_chunk is the position
// of the chunk's first token and n its valid rows (rows past it give zeros).
// Row 2 prb takes the hardware sine and cosine of its own angle, reduced in
// fp64 to a fraction of a turn; rows 2 prb + 1, + 32 and + 33 turn it by one,
// 32 and 33 positions with per-frequency constants. Each row's values are
// formed just before its pieces use them. The reduced angles of the wave's
// four rows go through LDS at base + PRO_BASE + 1024 w (lane l computes
// frequency l of each) and are read back by the same wave (its LDS accesses
// complete in order).
template <bool Q>
__device__ __forceinline__ void prologue_chunk(u32x4 (&kr)[2][2], u32x4 (&qr)[2][2], char *lds,
                                               int base, int64_t pos_chunk, int n, float eps,
                                               int tidv) {
    const int w = tidv >> 6;
    const int cidx = tidv & 15;
    const int prb = (tidv >> 4) & 15;  // 4 w + (lane >> 4)
    const int wb = base + PRO_BASE + 1024 * w;
    {
        const double om = lds_ld<double>(lds, base + PRO_OM + 8 * (tidv & 63));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            lds_st(lds, wb + 256 * j + 4 * (tidv & 63),
                   rope_base_turns(pos_chunk + 2 * (4 * w + j), om));
    }
    const int fb = 4 * 8 * (cidx & 7);
    const int rb = wb + 256 * ((tidv >> 4) & 3);
    const float4 b0 = lds_ld<float4>(lds, rb + fb), b1 = lds_ld<float4>(lds, rb + fb + 16);
    // The lower half of the row turns its partner in with a minus sign:
    // there every sine is negated (the angle is).
    const float sg = cidx >= 8 ? 1.f : -1.f;
    const float bt[8] = {sg * b0.x, sg * b0.y, sg * b0.z, sg * b0.w,
                         sg * b1.x, sg * b1.y, sg * b1.z, sg * b1.w};
    float c0[8], s0[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        c0[e] = cos_turns(bt[e]);
        s0[e] = sin_turns(bt[e]);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            float cs[8], sn[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float c = c0[e], sv = s0[e];
                if (it) {
                    const float2 r32 = lds_ld<float2>(lds, base + PRO_ROT32 + 2 * fb + 8 * e);
                    const float rs = sg * r32.y;
                    const float cn = fmaf(c, r32.x, -sv * rs);
                    sv = fmaf(sv, r32.x, c * rs);
                    c = cn;
                }
                if (rr) {
                    const float2 rot = lds_ld<float2>(lds, base + PRO_ROT + 2 * fb + 8 * e);
                    const float rs = sg * rot.y;
                    const float cn = fmaf(c, rot.x, -sv * rs);
                    sv = fmaf(sv, rot.x, c * rs);
                    c = cn;
                }
                cs[e] = c;
                sn[e] = sv;
            }
            const int r = 2 * (prb + 16 * it) + rr;
            kr[it][rr] = qk_prologue_piece(kr[it][rr], lds, base + PRO_W + 512 + 32 * cidx, cs, sn,
                                           r < n, eps);
            if (Q)
                qr[it][rr] = qk_prologue_piece(qr[it][rr], lds, base + PRO_W + 32 * cidx, cs, sn,
                                               r < n, eps);
        }
}

template <bool STATE_ONLY, bool PRO>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void chunk_mfma_kernel(ChunkParams p) {
    const int s = blockIdx.x / p.H;
    const int h = blockIdx.x - s * p.H;
    if (s >= p.nseg_max) return;
    const SegEntry se = seg_at(p, s);
    if (se.len < 0) return;
    const bool last = se.p == se.nseg - 1;
    // The state pass skips the segments of each sequence's last output
    // segment (rsub of them): nothing after them needs their states.
    if (STATE_ONLY && se.p >= p.rsub * ((se.nseg + p.rsub - 1) / p.rsub - 1)) return;

    constexpr int kBase = STATE_ONLY ? LDS_STATE : LDS_OUT;
    __shared__ __attribute__((aligned(16))) char lds[kBase + (PRO ? PRO_BYTES : 0)];
    const int offKT = STATE_ONLY ? 0 : OFF_KT;
    const int offVT = STATE_ONLY ? 16384 : OFF_VT;

    const int H = p.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const uint16_t *__restrict__ qg = static_cast<const uint16_t *>(p.q);
    const uint16_t *__restrict__ kg = static_cast<const uint16_t *>(p.k);
    const uint16_t *__restrict__ vg = static_cast<const uint16_t *>(p.v);
    uint16_t *__restrict__ og = static_cast<uint16_t *>(p.out);
    const int64_t sl = (int64_t)D * D;

    // The carried-in state in accumulator layout.
    f32x16 S[4];
    {
        const float *src = nullptr;
        if (!STATE_ONLY) {
            if (se.nseg == 1) src = p.s0 ? p.s0 + ((int64_t)se.seq * H + h) * sl : nullptr;
            else src = p.buf + ((int64_t)s * H + h) * sl;
        }
        if (src) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int dk = 32 * b + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
                    S[b][v] = src[dk * D + 32 * w + (l & 31)];
                }
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b) S[b] = f32x16{};
        }
    }

    // Each thread moves two row pairs of 16-byte chunks per tile:
    // pair pr = (tid >> 4) + 16 * it, rows 2pr and 2pr+1, chunk cidx.
    u32x4 qr[2][2] = {}, kr[2][2] = {}, vr[2][2] = {};
    float gr = 0.f;
    // Byte offset of this thread's 16-byte piece of row r inside a chunk, the
    // same for q, k, v and out ([T, H, 128] rows of 256 bytes): 32-bit per
    // lane on top of a per-chunk uniform base.
    auto piece = [&](int r, int tv) -> uint32_t {
        return (uint32_t)(r * H) * (uint32_t)(D * 2) + (uint32_t)(tv & 15) * 16u;
    };
    // Bytes from a chunk's first row to the end of its row n - 1 in q, k, v
    // and out: the range of the chunk's buffer resources, so that rows past
    // the end read as zeros and are not written (< 2^31 for H <= 65536).
    auto rows_bytes = [&](int n) -> int { return (n - 1) * H * (D * 2) + D * 2; };
    auto issue = [&](int64_t t0, int n) {
        // Opaque copy of the thread index: the per-lane offsets are rebuilt
        // here rather than kept across the loop.
        int tv = tid;
        asm volatile("" : "+v"(tv));
        const int64_t base = (t0 * H + h) * D;
        const int nb = rows_bytes(n);
        const buf_t rq = buf_rsrc(qg + base, nb);
        const buf_t rk = buf_rsrc(kg + base, nb);
        const buf_t rv = buf_rsrc(vg + base, nb);
        gr = buf_ld_f32(buf_rsrc(p.g + t0 * H + h, (n - 1) * H * 4 + 4), (tv & 63) * H * 4);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const uint32_t off = piece(2 * (((tv >> 4) & 15) + 16 * it) + rr, tv);
                kr[it][rr] = buf_ld16(rk, off);
                vr[it][rr] = buf_ld16(rv, off);
                if (!STATE_ONLY) qr[it][rr] = buf_ld16(rq, off);
            }
    };

    // Prologue tables, and the position of the segment's first token.
    int64_t pos0 = 0;
    if (PRO) {
        prologue_tables(lds, kBase, STATE_ONLY ? nullptr : p.qw, p.kw, p.theta, tid);
        pos0 = (p.pos_off ? (int64_t)p.pos_off[se.seq] : 0) + (int64_t)se.p * p.seg_len;
        __syncthreads();
    }

    const int len = se.len;
    if (len > 0) issue(se.tok0, min(64, len));
    // Everything loaded so far completes before the loop. The loop's own waits
    // then cover only the next chunk's loads, and the output stores issued
    // after them stay in flight across the loop's back edge.
    settle(gr);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            settle(kr[it][rr]);
            settle(vr[it][rr]);
            if (!STATE_ONLY) settle(qr[it][rr]);
        }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) settle(S[b][v]);
    float gam_acc = 0.f;

    // Two output workgroups share each CU, one from each half of the grid when
    // the grid fills the chip once, and when both have a wave ready the SIMD
    // picks the older one: left alone, the first-dispatched workgroup ends its
    // loop about 6 us before the other. Alternating a raised wave priority
    // between the two halves chunk by chunk lets each lead in turn.
    const int half = blockIdx.x >= gridDim.x / 2 ? 1 : 0;
    for (int c0 = 0; c0 < len; c0 += 64) {
        if (!STATE_ONLY) {
            if (((c0 >> 6) + half) & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        const int n = min(64, len - c0);
        const int64_t t0 = se.tok0 + c0;
        // The swizzled LDS addresses depend on the lane; rebuilding them from
        // an opaque copy of the thread index each chunk keeps the compiler from
        // holding ~80 of them in registers across the loop.
        int tidv = tid;
        asm volatile("" : "+v"(tidv));
        const int ln = tidv & 31;
        const int lh = (tidv >> 5) & 1;
        const int cidx = tidv & 15;
        const int prb = (tidv >> 4) & 15;

        // Gate prefix sum, one lane per token, in every wave.
        const float G = wave_prefix_sum(gr);
        const float Gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
        gam_acc += Gl;
        float fac[2][2];
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
                fac[it][rr] = __expf(Gl - __shfl(G, 2 * (prb + 16 * it) + rr, 64));

        if (PRO) prologue_chunk<!STATE_ONLY>(kr, qr, lds, kBase, pos0 + c0, n, p.eps, tidv);

        __syncthreads();  // every reader of the previous chunk's tiles is done
        if (!STATE_ONLY) {
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = 2 * (prb + 16 * it) + rr;
                    lds_st(lds, OFF_Q + row_off(r, cidx), qr[it][rr]);
                    lds_st(lds, OFF_K + row_off(r, cidx), kr[it][rr]);
                }
            if (w == 0) lds_st(lds, OFF_G + 4 * l, G);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int r0 = 2 * (prb + 16 * it);
            const int cb = (r0 & 7) * 2;  // byte offset of the token pair inside its chunk
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t a0 = vr[it][0][e2], a1 = vr[it][1][e2];
                const int d = 8 * cidx + 2 * e2;
                lds_st(lds, offVT + tr_off(d, r0 >> 3) + cb, pack_lo(a0, a1));
                lds_st(lds, offVT + tr_off(d + 1, r0 >> 3) + cb, pack_hi(a0, a1));
                const uint32_t k0 = kr[it][0][e2], k1 = kr[it][1][e2];
                lds_st(lds, offKT + tr_off(d, r0 >> 3) + cb,
                       pack_f32(lo_bf16(k0) * fac[it][0], lo_bf16(k1) * fac[it][1]));
                lds_st(lds, offKT + tr_off(d + 1, r0 >> 3) + cb,
                       pack_f32(hi_bf16(k0) * fac[it][0], hi_bf16(k1) * fac[it][1]));
            }
        }
        __syncthreads();  // tiles of this chunk are in LDS

        if (c0 + 64 < len) issue(t0 + 64, min(64, len - c0 - 64));

        // V operand (lane: value column 32w+ln, 8 tokens), shared by V^T A^T and the update.
        bf16x8 vop[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) vop[st] = lds_ld<bf16x8>(lds, offVT + tr_off(32 * w + ln, 2 * st + lh));

        if (!STATE_ONLY) {
            // Scores: wave 0 -> (j 0-31, i 0-31), 1 -> (j 0-31, i 32-63), 2 -> (j 32-63, i 32-63).
            if (w < 3) {
                const int jb = w == 2 ? 1 : 0;
                const int ib = w == 0 ? 0 : 1;
                f32x16 acc = {};
                const int j = 32 * jb + ln;
                const int i = 32 * ib + ln;
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const bf16x8 a = lds_ld<bf16x8>(lds, OFF_K + row_off(j, 2 * st + lh));
                    const bf16x8 bq = lds_ld<bf16x8>(lds, OFF_Q + row_off(i, 2 * st + lh));
                    acc = mfma(a, bq, acc);
                }
                const float Gi = lds_ld<float>(lds, OFF_G + 4 * i);
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int jr = 32 * jb + 8 * g4 + 4 * lh;
                    const float4 Gj = lds_ld<float4>(lds, OFF_G + 4 * jr);
                    const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
                    float val[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        val[r] = (jr + r <= i) ? p.scale * __expf(Gi - gj[r]) * acc[4 * g4 + r] : 0.f;
                    u32x2 pk = {pack_f32(val[0], val[1]), pack_f32(val[2], val[3])};
                    lds_st(lds, OFF_A + tr_off(i, 4 * jb + g4) + 8 * lh, pk);
                }
            }
            __syncthreads();  // A complete; K rows free for the O staging

            // O^T = S^T Q^T for both token halves, each state tile converted
            // once to the bf16 pair hi + lo.
            f32x16 acc[2] = {};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    bf16x8 sh, sl;
                    {
                        float x[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = S[b][8 * s2 + e];
                        split_bf16x8(x, sh, sl);
                    }
                    const int c = 4 * b + 2 * s2;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int i = 32 * nt + ln;
                        const bf16x4 x0 = lds_ld<bf16x4>(lds, OFF_Q + row_off(i, c) + 8 * lh);
                        const bf16x4 x1 = lds_ld<bf16x4>(lds, OFF_Q + row_off(i, c + 1) + 8 * lh);
                        const bf16x8 bq = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                        acc[nt] = mfma(sh, bq, acc[nt]);
                        acc[nt] = mfma(sl, bq, acc[nt]);
                    }
                }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int i = 32 * nt + ln;
                const float f = p.scale * __expf(lds_ld<float>(lds, OFF_G + 4 * i));
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[nt][v] *= f;
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    if (nt == 0 && st >= 2) break;
                    const bf16x8 ba = lds_ld<bf16x8>(lds, OFF_A + tr_off(i, 2 * st + lh));
                    acc[nt] = mfma(vop[st], ba, acc[nt]);
                }
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    u32x2 pk = {pack_f32(acc[nt][4 * g4], acc[nt][4 * g4 + 1]),
                                pack_f32(acc[nt][4 * g4 + 2], acc[nt][4 * g4 + 3])};
                    lds_st(lds, OFF_K + row_off(i, 4 * w + g4) + 8 * lh, pk);
                }
            }
        }

        const bool need_update = STATE_ONLY || (c0 + 64 < len) || (last && p.sfin);
        if (need_update) {
            const float a = __expf(Gl);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
#pragma unroll
                for (int v = 0; v < 16; ++v) S[b][v] *= a;
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf16x8 ka = lds_ld<bf16x8>(lds, offKT + tr_off(32 * b + ln, 2 * st + lh));
                    S[b] = mfma(ka, vop[st], S[b]);
                }
            }
        }

        if (!STATE_ONLY) {
            __syncthreads();  // O staging rows complete
            const buf_t ro = buf_rsrc(og + (t0 * H + h) * D, rows_bytes(n));
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = 2 * (prb + 16 * it) + rr;
                    buf_st16_nt(ro, piece(r, tidv), lds_ld<u32x4>(lds, OFF_K + row_off(r, cidx)));
                }
        }
    }

    float *dst = nullptr;
    if (STATE_ONLY) dst = p.buf + ((int64_t)s * H + h) * sl;
    else if (last && p.sfin) dst = p.sfin + ((int64_t)se.seq * H + h) * sl;
    if (dst) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int dk = 32 * b + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
                dst[dk * D + 32 * w + (l & 31)] = S[b][v];
            }
    }
    if (STATE_ONLY && tid == 0) p.gam[(int64_t)s * H + h] = gam_acc;
}

// The segment-state pass over value-column halves (inputs without the q/k
// prologue): the state-only pass above, with one workgroup per (sub-segment,
// head, half of the value columns), laid out by xcd_unit_map so that the two
// halves of a sub-segment run on one XCD and read its k rows through that
// XCD's L2. Twice the workgroups of the one-level pass, each with half its
// MFMA and vector work per chunk: about two workgroups per compute unit, so
// that one's load latency hides behind the other's work. Wave w holds key
// rows 64 (w >> 1) .. + 63 and value columns 32 (w & 1) .. + 31 of the half,
// as two 32x32 accumulator tiles. The result, the sub-segment's state from a
// zero start and its total log-decay, goes where the scan reads it, as from
// the one-level pass.
constexpr int SH_KT = 0;       // (K * exp(G_last - G))^T [128 dk][128 B]
constexpr int SH_VT = 16384;   // V^T of the half [64 dv][128 B]
constexpr int SH_BYTES = 24576;
static_assert(2 * SH_BYTES <= kLdsPerCU, "two state workgroups must fit one CU's LDS");

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void state_halves_kernel(ChunkParams p) {
    int unit, half;
    xcd_unit_map(blockIdx.x, 2, unit, half);
    const int H = p.H;
    const int s = unit / H;
    const int h = unit - s * H;
    if (s >= p.nseg_max) return;
    const SegEntry se = seg_at(p, s);
    if (se.len < 0) return;
    // The last output segment of a sequence needs no carried-out state.
    if (se.p >= p.rsub * ((se.nseg + p.rsub - 1) / p.rsub - 1)) return;
    __shared__ __attribute__((aligned(16))) char lds[SH_BYTES];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int cb = w & 1, kb = w >> 1;
    const uint16_t *__restrict__ kg = static_cast<const uint16_t *>(p.k);
    const uint16_t *__restrict__ vg = static_cast<const uint16_t *>(p.v);
    const int64_t sl = (int64_t)D * D;

    // This thread's share of a chunk: k pieces (tid & 15) of rows
    // 2 (((tid >> 4) & 15) + 16 it) + rr, v pieces (tid & 7) of the half of
    // rows 2 ((tid >> 3) & 31) + rr, and g of token (tid & 63); a buffer
    // range ending at the chunk's last row zeroes the rows past a ragged end.
    u32x4 kr[2][2], vr[2];
    float gr;
    auto rows_bytes = [&](int n) -> int { return (n - 1) * H * (D * 2) + D * 2; };
    auto issue = [&](int64_t t0, int n) {
        int tv = tid;
        asm volatile("" : "+v"(tv));
        const int64_t base = (t0 * H + h) * D;
        const int nb = rows_bytes(n);
        const buf_t rk = buf_rsrc(kg + base, nb);
        const buf_t rv = buf_rsrc(vg + base + 64 * half, nb - 128);
        gr = buf_ld_f32(buf_rsrc(p.g + t0 * H + h, (n - 1) * H * 4 + 4), (tv & 63) * H * 4);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = 2 * (((tv >> 4) & 15) + 16 * it) + rr;
                kr[it][rr] = buf_ld16(rk, (uint32_t)(r * H) * (uint32_t)(D * 2) + (uint32_t)(tv & 15) * 16u);
            }
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * ((tv >> 3) & 31) + rr;
            vr[rr] = buf_ld16(rv, (uint32_t)(r * H) * (uint32_t)(D * 2) + (uint32_t)(tv & 7) * 16u);
        }
    };

    f32x16 S[2] = {};
    float gam_acc = 0.f;
    const int len = se.len;
    if (len > 0) issue(se.tok0, min(64, len));
    for (int c0 = 0; c0 < len; c0 += 64) {
        const int64_t t0 = se.tok0 + c0;
        int tidv = tid;
        asm volatile("" : "+v"(tidv));
        const int ln = tidv & 31;
        const int lh = (tidv >> 5) & 1;
        const int cidx = tidv & 15;
        const int prb = (tidv >> 4) & 15;

        const float G = wave_prefix_sum(gr);
        const float Gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
        gam_acc += Gl;
        float fac[2][2];
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
                fac[it][rr] = __expf(Gl - __shfl(G, 2 * (prb + 16 * it) + rr, 64));

        __syncthreads();  // every reader of the previous chunk's tiles is done
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int r0 = 2 * (prb + 16 * it);
            const int bo = (r0 & 7) * 2;  // byte offset of the token pair inside its chunk
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t k0 = kr[it][0][e2], k1 = kr[it][1][e2];
                const int d = 8 * cidx + 2 * e2;
                lds_st(lds, SH_KT + tr_off(d, r0 >> 3) + bo,
                       pack_f32(lo_bf16(k0) * fac[it][0], lo_bf16(k1) * fac[it][1]));
                lds_st(lds, SH_KT + tr_off(d + 1, r0 >> 3) + bo,
                       pack_f32(hi_bf16(k0) * fac[it][0], hi_bf16(k1) * fac[it][1]));
            }
        }
        {
            const int r0 = 2 * ((tidv >> 3) & 31);
            const int bo = (r0 & 7) * 2;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t a0 = vr[0][e2], a1 = vr[1][e2];
                const int d = 8 * (tidv & 7) + 2 * e2;
                lds_st(lds, SH_VT + tr_off(d, r0 >> 3) + bo, pack_lo(a0, a1));
                lds_st(lds, SH_VT + tr_off(d + 1, r0 >> 3) + bo, pack_hi(a0, a1));
            }
        }
        __syncthreads();  // tiles of this chunk are in LDS

        if (c0 + 64 < len) issue(t0 + 64, min(64, len - c0 - 64));

        bf16x8 vop[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) vop[st] = lds_ld<bf16x8>(lds, SH_VT + tr_off(32 * cb + ln, 2 * st + lh));
        const float a = __expf(Gl);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int v = 0; v < 16; ++v) S[b][v] *= a;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 ka = lds_ld<bf16x8>(lds, SH_KT + tr_off(64 * kb + 32 * b + ln, 2 * st + lh));
                S[b] = mfma(ka, vop[st], S[b]);
            }
        }
    }

    float *dst = p.buf + ((int64_t)s * H + h) * sl;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int dk = 64 * kb + 32 * b + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
            dst[dk * D + 64 * half + 32 * cb + (l & 31)] = S[b][v];
        }
    if (half == 0 && tid == 0) p.gam[(int64_t)s * H + h] = gam_acc;
}

// The prologue alone: one workgroup per (64-token chunk, head) of x [B, T,
// H, 128] bf16, through the same loads and the same prologue_chunk as the
// chunked kernels; token t of sequence b sits at position pos_off[b] + t.
__global__ __launch_bounds__(NT) void qk_norm_rope_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const int32_t *__restrict__ pos_off,
                                                          uint16_t *out, int B, int T, int H,
                                                          float theta, float eps) {
    __shared__ __attribute__((aligned(16))) char lds[PRO_BYTES];
    const int64_t unit = blockIdx.x;
    const int h = (int)(unit % H);
    const int64_t bc = unit / H;
    const int nch = (T + 63) / 64;
    const int b = (int)(bc / nch);
    const int c = (int)(bc - (int64_t)b * nch);
    if (b >= B) return;
    const int tid = threadIdx.x;
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int n = min(64, T - 64 * c);
    const int64_t base = (((int64_t)b * T + 64 * (int64_t)c) * H + h) * D;
    const int nb = (n - 1) * H * (D * 2) + D * 2;
    const buf_t rx = buf_rsrc(x + base, nb);
    const buf_t ro = buf_rsrc(out + base, nb);
    u32x4 kr[2][2], none[2][2];
    auto off = [&](int it, int rr) -> uint32_t {
        const int r = 2 * (((tidv >> 4) & 15) + 16 * it) + rr;
        return (uint32_t)(r * H) * (uint32_t)(D * 2) + (uint32_t)(tidv & 15) * 16u;
    };
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) kr[it][rr] = buf_ld16(rx, off(it, rr));
    prologue_tables(lds, 0, nullptr, w, theta, tid);
    __syncthreads();
    const int64_t pos = (pos_off ? (int64_t)pos_off[b] : 0) + 64 * (int64_t)c;
    prologue_chunk<false>(kr, none, lds, 0, pos, n, eps, tidv);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) buf_st16(ro, off(it, rr), kr[it][rr]);
}

}  // namespace

hipError_t launch_qk_norm_rope(const void *x, const float *w, const int32_t *pos_off, void *out,
                               int B, int T, int H, float theta, float eps, hipStream_t st) {
    const int64_t units = (int64_t)B * ((T + 63) / 64) * H;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)units), dim3(NT), 0, st,
                       static_cast<const uint16_t *>(x), w, pos_off, static_cast<uint16_t *>(out),
                       B, T, H, theta, eps);
    return hipGetLastError();
}

hipError_t launch_chunk_mfma(const ChunkParams &p, bool phase_state, hipStream_t st) {
    if (p.nseg_max == 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.nseg_max * p.H));
    if (p.qw) {
        if (phase_state) hipLaunchKernelGGL((chunk_mfma_kernel<true, true>), grid, dim3(NT), 0, st, p);
        else hipLaunchKernelGGL((chunk_mfma_kernel<false, true>), grid, dim3(NT), 0, st, p);
    } else {
        if (phase_state && p.state_halves) {
            // Two workgroups per (sub-segment, head), laid out by
            // xcd_unit_map: the grid covers every unit when it is a multiple
            // of 16.
            const int64_t units = (int64_t)p.nseg_max * p.H;
            hipLaunchKernelGGL(state_halves_kernel, dim3((unsigned)((2 * units + 15) / 16 * 16)), dim3(NT), 0, st, p);
        } else if (phase_state) {
            hipLaunchKernelGGL((chunk_mfma_kernel<true, false>), grid, dim3(NT), 0, st, p);
        } else {
            hipLaunchKernelGGL((chunk_mfma_kernel<false, false>), grid, dim3(NT), 0, st, p);
        }
    }
    return hipGetLastError();
}

}  // namespace sgla
