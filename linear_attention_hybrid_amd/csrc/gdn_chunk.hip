// Chunked gated delta rule (GDN) on the matrix cores: bf16 q, k, v, fp32
// gates g and write strengths beta, Dk = Dv = 128, chunks of 64 tokens, fp32
// state.
//
// Per chunk (page "Formulas and code for adapting inference to GDN/KDA linear
// modules", section 1.2, the chunkwise formulas), with G the inclusive
// cumulative sum of g inside the chunk and Gamma[i][j] = exp(G_i - G_j):
//
//   A     = strictly_lower(diag(beta) K K^T * Gamma)
//   T     = (I + A)^-1                                     (UT transform)
//   W     = T diag(beta exp(G)) K ,   U = T diag(beta) V
//   new_v = U - W S
//   O     = scale ((Q * exp(G)) S + lower(Q K^T * Gamma) new_v)
//   S     = exp(G_last) S + (K * exp(G_last - G))^T new_v
//
// W and U depend on the chunk alone, so they are computed for every chunk at
// once by a first kernel (gdn_prep_kernel), one workgroup per (chunk, head),
// and kept in a workspace (W in bf16, an MFMA operand; U in fp32). The state
// recurrence is sequential over chunks: gdn_chunk_kernel walks one (sequence,
// head) per workgroup through its chunks with the fp32 state in the MFMA
// accumulators.
//
// Precision: the state is written through new_v, which is not a bf16 input
// (beta v already is not), so the update takes exp(G_last - G) new_v in fp32
// split into a bf16 high and low part against the exact bf16 K: the write
// into the state keeps about 16 bits. The output products use bf16 operands
// (state, scores, new_v) as the Simple GLA kernels do.
//
// The inverse T is found in fp32 by back substitution on (I + A)^T, whose
// solution for unit vector e_c is row c of T: lane c of one wave computes row
// c and writes it contiguously, 64 lanes, 64 rows, no transposition. The
// column scalings beta exp(G) and beta are folded into T, which is then split
// into a bf16 high and low part, so W and U come from exact bf16 K and V
// times a T accurate to about 2^-16.
#include "mfma_tile.h"

namespace sgla {

namespace {

constexpr int D = 128;
constexpr int NT = 256;

// ---- gdn_prep_kernel LDS map (bytes).
constexpr int P_K = 0;             // K rows [64][256 B]; then T' high and low parts
constexpr int P_KT = 16384;        // K^T [128 dk][128 B]
constexpr int P_VT = 32768;        // V^T [128 dv][128 B]
constexpr int P_AT = 49152;        // A^T fp32 [64][68]; then T'' high and low parts
constexpr int AT_ROW = 68 * 4;     // padded row (16-byte aligned, rows start 4 banks apart)
constexpr int P_G = P_AT + 64 * AT_ROW;
constexpr int P_B = P_G + 256;
constexpr int P_BYTES = P_B + 256;
constexpr int P_TPH = 0;           // T' = T diag(beta exp(G)), [64 rows][128 B] bf16, high part
constexpr int P_TPL = 8192;        // low part
constexpr int P_TQH = P_AT;        // T'' = T diag(beta), high part
constexpr int P_TQL = P_AT + 8192; // low part
static_assert(P_TQL + 8192 <= P_G, "T'' parts overlap the gate tables");

// ---- gdn_chunk_kernel LDS map (bytes).
constexpr int C_Q = 0;       // Q rows [64][256 B]
constexpr int C_K = 16384;   // K rows [64][256 B]; later the O staging rows
constexpr int C_KT = 32768;  // K^T [128 dk][128 B]
constexpr int C_W = 49152;   // W rows [64][256 B]
constexpr int C_A = 65536;   // scores A[64 i][128 B]
constexpr int C_G = 73728;   // G[64] fp32
constexpr int C_BYTES = C_G + 256;

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__global__ __launch_bounds__(NT) void gdn_prep_kernel(GdnParams p) {
    const int H = p.c.H;
    const int s = blockIdx.x / H;
    const int h = blockIdx.x - s * H;
    if (s >= p.c.nseg_max) return;
    const SegEntry se = seg_at(p.c, s);
    if (se.len <= 0) return;
    const int n = se.len;  // <= 64
    __shared__ __attribute__((aligned(16))) char lds[P_BYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int ln = l & 31;
    const int lh = l >> 5;
    const int cidx = tid & 15;
    const int prb = (tid >> 4) & 15;

    // K and V rows: each thread moves two row pairs of 16-byte pieces.
    const int64_t base = (se.tok0 * H + h) * D;
    const uint16_t *kg = static_cast<const uint16_t *>(p.c.k) + base;
    const uint16_t *vg = static_cast<const uint16_t *>(p.c.v) + base;
    const int64_t row_stride = (int64_t)H * D;
    u32x4 kr[2][2], vr[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * (prb + 16 * it) + rr;
            const bool ok = r < n;
            kr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(kg + r * row_stride + 8 * cidx) : u32x4{0, 0, 0, 0};
            vr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(vg + r * row_stride + 8 * cidx) : u32x4{0, 0, 0, 0};
        }
    const float gv = l < n ? p.c.g[(se.tok0 + l) * H + h] : 0.f;
    const float bv = l < n ? p.beta[(se.tok0 + l) * H + h] : 0.f;
    const float G = wave_prefix_sum(gv);
    if (w == 0) {
        lds_st(lds, P_G + 4 * l, G);
        lds_st(lds, P_B + 4 * l, bv);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
            lds_st(lds, P_K + row_off(2 * (prb + 16 * it) + rr, cidx), kr[it][rr]);
        const int r0 = 2 * (prb + 16 * it);
        const int cb = (r0 & 7) * 2;  // byte offset of the token pair inside its 8-token piece
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const int d = 8 * cidx + 2 * e2;
            const uint32_t k0 = kr[it][0][e2], k1 = kr[it][1][e2];
            const uint32_t v0 = vr[it][0][e2], v1 = vr[it][1][e2];
            lds_st(lds, P_KT + tr_off(d, r0 >> 3) + cb, pack_lo(k0, k1));
            lds_st(lds, P_KT + tr_off(d + 1, r0 >> 3) + cb, pack_hi(k0, k1));
            lds_st(lds, P_VT + tr_off(d, r0 >> 3) + cb, pack_lo(v0, v1));
            lds_st(lds, P_VT + tr_off(d + 1, r0 >> 3) + cb, pack_hi(v0, v1));
        }
    }
    __syncthreads();

    // A^T[m][i] = A[i][m] = beta_i (k_i . k_m) exp(G_i - G_m) for i > m, else 0.
    // Waves 0-2 take the tiles (i block, m block) = (0,0), (1,0), (1,1); the
    // tile with every i < m is never read.
    if (w < 3) {
        const int ib = w == 0 ? 0 : 1;
        const int mb = w == 2 ? 1 : 0;
        const int ir = 32 * ib + ln;
        const int m = 32 * mb + ln;
        f32x16 acc = {};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const bf16x8 a = lds_ld<bf16x8>(lds, P_K + row_off(ir, 2 * st + lh));
            const bf16x8 b = lds_ld<bf16x8>(lds, P_K + row_off(m, 2 * st + lh));
            acc = mfma(a, b, acc);
        }
        const float Gm = lds_ld<float>(lds, P_G + 4 * m);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int i0 = 32 * ib + 8 * g4 + 4 * lh;
            const float4 Gi = lds_ld<float4>(lds, P_G + 4 * i0);
            const float4 Bi = lds_ld<float4>(lds, P_B + 4 * i0);
            const float gi[4] = {Gi.x, Gi.y, Gi.z, Gi.w};
            const float bi[4] = {Bi.x, Bi.y, Bi.z, Bi.w};
            float a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a[r] = (i0 + r > m) ? bi[r] * acc[4 * g4 + r] * __expf(gi[r] - Gm) : 0.f;
            lds_st(lds, P_AT + m * AT_ROW + 4 * i0, make_float4(a[0], a[1], a[2], a[3]));
        }
    }
    __syncthreads();

    // Row c = l of T = (I + A)^-1 by back substitution on (I + A)^T y = e_c:
    // y_m = [m == c] - sum_{j > m} A[j][m] y_j, for m = 63 down to 0.
    if (w == 0) {
        float y[64];
#pragma unroll
        for (int m = 63; m >= 0; --m) {
            float acc = m == l ? 1.f : 0.f;
#pragma unroll
            for (int jq = (m + 1) & ~3; jq < 64; jq += 4) {
                const float4 a = lds_ld<float4>(lds, P_AT + m * AT_ROW + 4 * jq);
                if (jq + 0 > m) acc = fmaf(-a.x, y[jq + 0], acc);
                if (jq + 1 > m) acc = fmaf(-a.y, y[jq + 1], acc);
                if (jq + 2 > m) acc = fmaf(-a.z, y[jq + 2], acc);
                if (jq + 3 > m) acc = fmaf(-a.w, y[jq + 3], acc);
            }
            y[m] = acc;
        }
        // T'[c][m] = y_m beta_m exp(G_m), T''[c][m] = y_m beta_m, each as a
        // bf16 high part and the bf16 rounding of the rest.
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 G0 = lds_ld<float4>(lds, P_G + 32 * q);
            const float4 G1 = lds_ld<float4>(lds, P_G + 32 * q + 16);
            const float4 B0 = lds_ld<float4>(lds, P_B + 32 * q);
            const float4 B1 = lds_ld<float4>(lds, P_B + 32 * q + 16);
            const float gq[8] = {G0.x, G0.y, G0.z, G0.w, G1.x, G1.y, G1.z, G1.w};
            const float bq[8] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
            bf16x8 ph, pl, qh, ql;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float tq = y[8 * q + e] * bq[e];
                const float tp = tq * __expf(gq[e]);
                ph[e] = (__bf16)tp;
                pl[e] = (__bf16)(tp - (float)ph[e]);
                qh[e] = (__bf16)tq;
                ql[e] = (__bf16)(tq - (float)qh[e]);
            }
            lds_st(lds, P_TPH + tr_off(l, q), ph);
            lds_st(lds, P_TPL + tr_off(l, q), pl);
            lds_st(lds, P_TQH + tr_off(l, q), qh);
            lds_st(lds, P_TQL + tr_off(l, q), ql);
        }
    }
    __syncthreads();

    // Wave w: W^T = K^T T'^T for dk rows [32w, 32w + 32) (stored as W rows,
    // token-major), and U = T'' V for value columns [32w, 32w + 32) (stored
    // as U^T rows, value-major, fp32). Rows past the chunk's end come out zero.
    uint16_t *wt = p.w + ((int64_t)s * H + h) * (64 * D);
    float *ut = p.u + ((int64_t)s * H + h) * (64 * D);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        f32x16 aw = {}, au = {};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8 kt = lds_ld<bf16x8>(lds, P_KT + tr_off(32 * w + ln, 2 * st + lh));
            const bf16x8 vt = lds_ld<bf16x8>(lds, P_VT + tr_off(32 * w + ln, 2 * st + lh));
            const int ti = 32 * nt + ln;
            aw = mfma(kt, lds_ld<bf16x8>(lds, P_TPH + tr_off(ti, 2 * st + lh)), aw);
            aw = mfma(kt, lds_ld<bf16x8>(lds, P_TPL + tr_off(ti, 2 * st + lh)), aw);
            au = mfma(lds_ld<bf16x8>(lds, P_TQH + tr_off(ti, 2 * st + lh)), vt, au);
            au = mfma(lds_ld<bf16x8>(lds, P_TQL + tr_off(ti, 2 * st + lh)), vt, au);
        }
        const int i = 32 * nt + ln;
        const int dv = 32 * w + ln;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 pw = {pack_f32(aw[4 * g4], aw[4 * g4 + 1]), pack_f32(aw[4 * g4 + 2], aw[4 * g4 + 3])};
            *reinterpret_cast<u32x2 *>(wt + i * D + 32 * w + 8 * g4 + 4 * lh) = pw;
            *reinterpret_cast<float4 *>(ut + dv * 64 + 32 * nt + 8 * g4 + 4 * lh) =
                make_float4(au[4 * g4], au[4 * g4 + 1], au[4 * g4 + 2], au[4 * g4 + 3]);
        }
    }
}

// One (sequence, head) per workgroup, through all its chunks. Wave w owns
// value columns [32w, 32w + 32) of the state (lane l: column 32w + l % 32,
// key rows 32b + 8(v/4) + 4(l/32) + v%4 of accumulator S[b], element v).
//
// new_v = U - W S comes out of the MFMA with each lane holding one value
// column and, per group of four, four consecutive tokens: converted in
// registers it is directly the token-indexed operand of the output product
// (bf16) and of the state update (exp(G_last - G) new_v as bf16 high and low
// parts), the other operand (scores, K^T) being read in the same token order.
__global__ __launch_bounds__(NT) void gdn_chunk_kernel(GdnParams p) {
    const int H = p.c.H;
    const int seq = blockIdx.x / H;
    const int h = blockIdx.x - seq * H;
    if (seq >= p.c.N) return;
    const SeqEntry sq = seq_at(p.c, seq);
    __shared__ __attribute__((aligned(16))) char lds[C_BYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const uint16_t *__restrict__ qg = static_cast<const uint16_t *>(p.c.q);
    const uint16_t *__restrict__ kg = static_cast<const uint16_t *>(p.c.k);
    uint16_t *__restrict__ og = static_cast<uint16_t *>(p.c.out);
    const int64_t sl = (int64_t)D * D;

    f32x16 S[4];
    {
        const float *src = p.c.s0 ? p.c.s0 + ((int64_t)seq * H + h) * sl : nullptr;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int dk = 32 * b + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
                S[b][v] = src ? src[dk * D + 32 * w + (l & 31)] : 0.f;
            }
    }

    u32x4 qr[2][2], kr[2][2], wr[2][2];
    float4 ur[2][4];
    float gr = 0.f;
    auto issue = [&](int j) {
        const SegEntry e = seg_at(p.c, sq.first + j);
        const int n = e.len;
        int tv = tid;
        asm volatile("" : "+v"(tv));
        const int64_t base = (e.tok0 * H + h) * D;
        const uint16_t *qb = qg + base;
        const uint16_t *kb = kg + base;
        const int64_t tile = ((int64_t)(sq.first + j) * H + h) * (64 * D);
        const uint16_t *wb = p.w + tile;
        const float *ub = p.u + tile;
        const int64_t rs = (int64_t)H * D;
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = 2 * (((tv >> 4) & 15) + 16 * it) + rr;
                const int c8 = 8 * (tv & 15);
                const bool ok = r < n;
                qr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(qb + r * rs + c8) : u32x4{0, 0, 0, 0};
                kr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(kb + r * rs + c8) : u32x4{0, 0, 0, 0};
                wr[it][rr] = *reinterpret_cast<const u32x4 *>(wb + r * D + c8);
            }
        // U^T pieces in accumulator order: value column 32w + l%32, tokens
        // 32nt + 8q + 4(l/32) .. + 3.
        const int dv = 32 * (tv >> 6) + (tv & 31);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                ur[nt][q] = *reinterpret_cast<const float4 *>(ub + dv * 64 + 32 * nt + 8 * q + 4 * ((tv >> 5) & 1));
        gr = (tv & 63) < n ? p.c.g[(e.tok0 + (tv & 63)) * H + h] : 0.f;
    };

    // nseg is at least 1 for a valid table (an empty sequence has one empty
    // row); offsets that break the rules can leave 0, and then no row is read.
    const int nch = sq.nseg;
    const bool any = nch > 1 || (nch == 1 && seg_at(p.c, sq.first).len > 0);
    if (any) issue(0);

    for (int j = 0; any && j < nch; ++j) {
        const SegEntry se = seg_at(p.c, sq.first + j);
        const int n = se.len;
        const int64_t t0 = se.tok0;
        int tidv = tid;
        asm volatile("" : "+v"(tidv));
        const int ln = tidv & 31;
        const int lh = (tidv >> 5) & 1;
        const int cidx = tidv & 15;
        const int prb = (tidv >> 4) & 15;

        const float G = wave_prefix_sum(gr);
        const float Gl = lane_value(G, 63);
        // U of this chunk, before the next chunk's loads reuse the registers.
        float uc[2][16];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uc[nt][4 * q + 0] = ur[nt][q].x;
                uc[nt][4 * q + 1] = ur[nt][q].y;
                uc[nt][4 * q + 2] = ur[nt][q].z;
                uc[nt][4 * q + 3] = ur[nt][q].w;
            }

        __syncthreads();  // every reader of the previous chunk's tiles is done
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = 2 * (prb + 16 * it) + rr;
                lds_st(lds, C_Q + row_off(r, cidx), qr[it][rr]);
                lds_st(lds, C_K + row_off(r, cidx), kr[it][rr]);
                lds_st(lds, C_W + row_off(r, cidx), wr[it][rr]);
            }
        if (w == 0) lds_st(lds, C_G + 4 * l, G);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int r0 = 2 * (prb + 16 * it);
            const int cb = (r0 & 7) * 2;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t k0 = kr[it][0][e2], k1 = kr[it][1][e2];
                const int d = 8 * cidx + 2 * e2;
                lds_st(lds, C_KT + tr_off(d, r0 >> 3) + cb, pack_lo(k0, k1));
                lds_st(lds, C_KT + tr_off(d + 1, r0 >> 3) + cb, pack_hi(k0, k1));
            }
        }
        __syncthreads();  // tiles of this chunk are in LDS

        if (j + 1 < nch) issue(j + 1);

        // The state as bf16 operands: B of W S (columns = value columns) and
        // A of S^T Q^T (rows = value columns), key rows in accumulator order.
        bf16x8 sb[4][2];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int e = 0; e < 8; ++e) sb[b][s2][e] = (__bf16)S[b][8 * s2 + e];

        // Scores: wave 0 -> (j 0-31, i 0-31), 1 -> (j 0-31, i 32-63), 2 -> (j 32-63, i 32-63).
        if (w < 3) {
            const int jb = w == 2 ? 1 : 0;
            const int ib = w == 0 ? 0 : 1;
            f32x16 acc = {};
            const int jj = 32 * jb + ln;
            const int i = 32 * ib + ln;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const bf16x8 a = lds_ld<bf16x8>(lds, C_K + row_off(jj, 2 * st + lh));
                const bf16x8 bq = lds_ld<bf16x8>(lds, C_Q + row_off(i, 2 * st + lh));
                acc = mfma(a, bq, acc);
            }
            const float Gi = lds_ld<float>(lds, C_G + 4 * i);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int jr = 32 * jb + 8 * g4 + 4 * lh;
                const float4 Gj = lds_ld<float4>(lds, C_G + 4 * jr);
                const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
                float val[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    val[r] = (jr + r <= i) ? p.c.scale * __expf(Gi - gj[r]) * acc[4 * g4 + r] : 0.f;
                const u32x2 pk = {pack_f32(val[0], val[1]), pack_f32(val[2], val[3])};
                lds_st(lds, C_A + tr_off(i, 4 * jb + g4) + 8 * lh, pk);
            }
        }

        // new_v = U - W S for this wave's value columns, both token halves:
        // nvop in bf16 for the output; exp(G_last - G) new_v as high and low
        // bf16 parts (nvh, nvl) for the state update.
        bf16x8 nvop[4], nvh[4], nvl[4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int i = 32 * nt + ln;
            f32x16 acc = {};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int c = 4 * b + 2 * s2;
                    const bf16x4 x0 = lds_ld<bf16x4>(lds, C_W + row_off(i, c) + 8 * lh);
                    const bf16x4 x1 = lds_ld<bf16x4>(lds, C_W + row_off(i, c + 1) + 8 * lh);
                    acc = mfma(cat4(x0, x1), sb[b][s2], acc);
                }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // tokens 32nt + 8q + 4(l/32) + r of accumulator element 4q + r
                const float4 Gt = lds_ld<float4>(lds, C_G + 4 * (32 * nt + 8 * q + 4 * lh));
                const float gt[4] = {Gt.x, Gt.y, Gt.z, Gt.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int v = 4 * q + r;
                    const float nv = uc[nt][v] - acc[v];
                    const float x = nv * __expf(Gl - gt[r]);
                    const __bf16 xh = (__bf16)x;
                    nvop[2 * nt + (v >> 3)][v & 7] = (__bf16)nv;
                    nvh[2 * nt + (v >> 3)][v & 7] = xh;
                    nvl[2 * nt + (v >> 3)][v & 7] = (__bf16)(x - (float)xh);
                }
            }
        }
        __syncthreads();  // scores complete; K rows free for the O staging

#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int i = 32 * nt + ln;
            f32x16 acc = {};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int c = 4 * b + 2 * s2;
                    const bf16x4 x0 = lds_ld<bf16x4>(lds, C_Q + row_off(i, c) + 8 * lh);
                    const bf16x4 x1 = lds_ld<bf16x4>(lds, C_Q + row_off(i, c + 1) + 8 * lh);
                    acc = mfma(sb[b][s2], cat4(x0, x1), acc);
                }
            const float f = p.c.scale * __expf(lds_ld<float>(lds, C_G + 4 * i));
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] *= f;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (nt == 0 && st >= 2) break;
                const bf16x4 y0 = lds_ld<bf16x4>(lds, C_A + tr_off(i, 2 * st) + 8 * lh);
                const bf16x4 y1 = lds_ld<bf16x4>(lds, C_A + tr_off(i, 2 * st + 1) + 8 * lh);
                acc = mfma(nvop[st], cat4(y0, y1), acc);
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const u32x2 pk = {pack_f32(acc[4 * g4], acc[4 * g4 + 1]),
                                  pack_f32(acc[4 * g4 + 2], acc[4 * g4 + 3])};
                lds_st(lds, C_K + row_off(i, 4 * w + g4) + 8 * lh, pk);
            }
        }

        const bool last = j + 1 == nch;
        if (!last || p.c.sfin) {
            const float a = __expf(Gl);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
#pragma unroll
                for (int v = 0; v < 16; ++v) S[b][v] *= a;
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf16x4 z0 = lds_ld<bf16x4>(lds, C_KT + tr_off(32 * b + ln, 2 * st) + 8 * lh);
                    const bf16x4 z1 = lds_ld<bf16x4>(lds, C_KT + tr_off(32 * b + ln, 2 * st + 1) + 8 * lh);
                    const bf16x8 kt = cat4(z0, z1);
                    S[b] = mfma(kt, nvh[st], S[b]);
                    S[b] = mfma(kt, nvl[st], S[b]);
                }
            }
        }

        __syncthreads();  // O staging rows complete
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = 2 * (prb + 16 * it) + rr;
                if (r < n) {
                    const u32x4 o = lds_ld<u32x4>(lds, C_K + row_off(r, cidx));
                    *reinterpret_cast<u32x4 *>(og + (t0 + r) * H * D + h * D + 8 * cidx) = o;
                }
            }
    }

    if (p.c.sfin) {
        float *dst = p.c.sfin + ((int64_t)seq * H + h) * sl;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int dk = 32 * b + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
                dst[dk * D + 32 * w + (l & 31)] = S[b][v];
            }
    }
}

}  // namespace

hipError_t launch_gdn_chunk(const GdnParams &p, hipStream_t st) {
    if (p.c.N == 0) return hipSuccess;
    if (p.c.nseg_max > 0)
        hipLaunchKernelGGL(gdn_prep_kernel, dim3((unsigned)((int64_t)p.c.nseg_max * p.c.H)), dim3(NT), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn_chunk_kernel, dim3((unsigned)((int64_t)p.c.N * p.c.H)), dim3(NT), 0, st, p);
    return hipGetLastError();
}

}  // namespace sgla
