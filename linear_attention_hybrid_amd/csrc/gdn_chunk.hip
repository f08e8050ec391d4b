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
// once by a first kernel (gdn_prep_kernel, persistent over the (chunk, head)
// items) and kept in a workspace (W in bf16, an MFMA operand; U in fp32). The state
// recurrence is sequential over chunks: gdn_chain_kernel walks each
// (sequence, head, block of 16 value columns) through its chunks with the
// fp32 state in the MFMA accumulators. A last kernel (gdn_output_kernel)
// forms every chunk's output at once from the states and new_v the chain
// leaves behind.
//
// Precision: the state is written through new_v, which is not a bf16 input
// (beta v already is not), so the update takes exp(G_last - G) new_v in fp32
// split into a bf16 high and low part against the exact bf16 K: the write
// into the state keeps about 16 bits. The output products use bf16 operands
// for the state and new_v, as the Simple GLA kernels do, and bf16 high and
// low parts for the scores.
//
// The inverse T is found in fp32 in 16 x 16 blocks. Each wave inverts one
// diagonal block by back substitution on its transpose, whose solution for
// unit vector e_r is row r of the block's inverse (right-looking: as soon as
// y_j is final it is taken out of every y_m, m < j; 15 dependent steps).
// The blocks below the diagonal follow block row by block row,
// T_IJ = -T_II sum_K A_IK T_KJ, on fp32 16 x 16 x 4 MFMAs. The column
// scalings beta exp(G) and beta are folded into T, which is then split into
// a bf16 high and low part, so W and U come from exact bf16 K and V times a
// T accurate to about 2^-16.
#include "mfma_tile.h"

namespace sgla {

namespace {

constexpr int D = 128;
constexpr int NT = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- gdn_prep_kernel LDS map (bytes).
constexpr int P_K = 0;             // K rows [64][256 B]; then T' high and low parts
constexpr int P_KT = 16384;        // K^T [128 dk][128 B]
constexpr int P_VT = 32768;        // V^T [128 dv][128 B]
constexpr int P_A = 49152;         // A fp32 [64][68], row-major; then T'' high and low parts
constexpr int A_ROW = 68 * 4;      // padded row (16-byte aligned, rows start 4 banks apart)
constexpr int P_G = P_A + 64 * A_ROW;
constexpr int P_B = P_G + 256;
constexpr int P_E = P_B + 256;     // exp(G) per token
constexpr int P_BYTES = P_E + 256;
static_assert(2 * P_BYTES <= kLdsPerCU, "two prep workgroups must fit one CU's LDS");
// T in 16 x 16 fp32 blocks (I, J), I >= J, rows of 80 bytes (20 floats: the
// 16 rows of a block start 4 banks apart), in the K rows region once K K^T
// is done.
constexpr int TB_ROW = 80;
constexpr int TB_BYTES = 16 * TB_ROW;
__host__ __device__ constexpr int tb_off(int I, int J) { return (I * (I + 1) / 2 + J) * TB_BYTES; }
static_assert(tb_off(3, 3) + TB_BYTES <= 16384, "T blocks exceed the K rows region");
constexpr int P_TPH = 0;           // T' = T diag(beta exp(G)), [64 rows][128 B] bf16, high part
constexpr int P_TPL = 8192;        // low part
constexpr int P_TQH = P_A;         // T'' = T diag(beta), high part
constexpr int P_TQL = P_A + 8192;  // low part
static_assert(P_TQL + 8192 <= P_G, "T'' parts overlap the gate tables");

// Per chunk and head the workspace tile holds W (16 KiB bf16 rows) and U
// (32 KiB fp32, as [slice w][piece p][lane l] x 16 B: lane l of piece p of
// slice w holds tokens 8p + 4(l/32) .. + 3 of value column 32w + l % 32).
// Slice w has the layout of the output kernel's operand image for its wave w
// (16 bytes per lane and operand, lanes consecutive), and the U of each chain
// workgroup (16 value columns: half the lanes of one slice) sits in exactly
// the bytes where that workgroup later stores its half of the chunk's start
// state, in bf16, as that image; no other workgroup reads them. The chunk's
// bf16 new_v goes, as an image too, to a separate 16 KiB per chunk and head.
constexpr int TILE_ELEMS = 64 * D;                 // bf16 elements of W; U is as many floats
constexpr int T_U = TILE_ELEMS * 2;                 // byte offset of U
constexpr int TILE_BYTES = 3 * TILE_ELEMS * 2;      // W + U = 48 KiB
constexpr int IMG_S = T_U;                          // state image: [block 4][8 operands][64 lanes] x 16 B
constexpr int NV_BYTES = 4 * 4 * 64 * 16;           // new_v image: [block 4][4 operands][64 lanes] x 16 B
static_assert(IMG_S + 4 * 8 * 64 * 16 == TILE_BYTES, "state image must fill the U slices");

__device__ __forceinline__ char *tile_at(const GdnParams &p, int64_t s, int h) {
    return p.tiles + ((int64_t)s * p.c.H + h) * TILE_BYTES;
}


// Persistent: workgroup b takes the (chunk, head) items b, b + gridDim.x, ...
// in chunk-major order, and loads the next item's k and v rows, g and beta
// into registers while it works on the current one, so that their latency is
// hidden behind that work.
__global__ __launch_bounds__(NT) void gdn_prep_kernel(GdnParams p, int nitems) {
    const int H = p.c.H;
    __shared__ __attribute__((aligned(16))) char lds[P_BYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int ln = l & 31;
    const int lh = l >> 5;
    const int cidx = tid & 15;
    const int prb = (tid >> 4) & 15;

    // An item's k and v rows (each thread two row pairs of 16-byte pieces;
    // zero past the chunk's end), g and beta.
    u32x4 kr[2][2], vr[2][2];
    float gv, bv;
    int fn;  // the fetched item's token count
    auto fetch = [&](int64_t item) {
        int n = 0, hh = 0;
        int64_t tok0 = 0;
        if (item < nitems) {
            const int s = (int)(item / H);
            hh = (int)(item - (int64_t)s * H);
            const SegEntry se = seg_at(p.c, s);
            n = se.len;
            tok0 = se.tok0;
        }
        // Buffer resources over the item's n rows: rows past the end (all of
        // them past the last item) read as zeros, with no branch around the
        // loads (< 2^31 bytes for H <= 65536).
        const int64_t base = (tok0 * H + hh) * D;
        const int nb = n > 0 ? (n - 1) * H * (D * 2) + D * 2 : 0;
        const buf_t rk = buf_rsrc(static_cast<const uint16_t *>(p.c.k) + base, nb);
        const buf_t rv = buf_rsrc(static_cast<const uint16_t *>(p.c.v) + base, nb);
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const uint32_t off = (uint32_t)((2 * (prb + 16 * it) + rr) * H) * (uint32_t)(D * 2) +
                                     16u * (uint32_t)cidx;
                kr[it][rr] = buf_ld16(rk, off);
                vr[it][rr] = buf_ld16_nt(rv, off);  // v: read only here
            }
        const int gb = n > 0 ? (n - 1) * H * 4 + 4 : 0;
        gv = buf_ld_f32(buf_rsrc(p.c.g + tok0 * H + hh, gb), (uint32_t)(l * H * 4));
        bv = buf_ld_f32(buf_rsrc(p.beta + tok0 * H + hh, gb), (uint32_t)(l * H * 4));
        fn = __builtin_amdgcn_readfirstlane(n);
    };

    fetch(blockIdx.x);
    // The first item's loads complete before the loop, so that the loop's own
    // waits cover only the next item's loads and not the W and U stores
    // issued after them.
    settle(gv);
    settle(bv);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            settle(kr[it][rr]);
            settle(vr[it][rr]);
        }
    // 64-bit, so that item + gridDim.x cannot wrap for item counts near 2^31.
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int s = (int)(item / H);
        const int h = (int)(item - (int64_t)s * H);
        const int n = fn;  // <= 64
        // Empty items (past the last one, or an empty table row) run the same
        // code on zeros, and their stores are dropped, so that every path
        // back to the loop top issues the same memory operations.
        const float G = wave_prefix_sum(gv);
        if (w == 0) {
            lds_st(lds, P_G + 4 * l, G);
            lds_st(lds, P_B + 4 * l, bv);
        } else if (w == 1) {
            lds_st(lds, P_E + 4 * l, __expf(G));
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
        fetch(item + gridDim.x);
        __syncthreads();

        // A[i][m] = beta_i (k_i . k_m) exp(G_i - G_m) for i > m, else 0, row-major,
        // as the ten 16 x 16 blocks (I, J), J <= I, spread over the four waves
        // (the blocks with J > I are never read). K K^T is symmetric; with the m
        // block as the A operand each lane holds one row i and four consecutive
        // m.
        {
            const int lc = l & 15;
            const int g = l >> 4;
            for (int bi = w; bi < 10; bi += 4) {
                const int I = bi >= 6 ? 3 : bi >= 3 ? 2 : bi >= 1 ? 1 : 0;
                const int J = bi - I * (I + 1) / 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 a = lds_ld<bf16x8>(lds, P_K + row_off(16 * J + lc, 4 * ks + g));
                    const bf16x8 b = lds_ld<bf16x8>(lds, P_K + row_off(16 * I + lc, 4 * ks + g));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
                }
                const int i = 16 * I + lc;
                const int m0 = 16 * J + 4 * g;
                const float Gi = lds_ld<float>(lds, P_G + 4 * i);
                const float bti = lds_ld<float>(lds, P_B + 4 * i);
                const float4 Gm = lds_ld<float4>(lds, P_G + 4 * m0);
                const float gm[4] = {Gm.x, Gm.y, Gm.z, Gm.w};
                float a[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a[r] = (i > m0 + r) ? bti * acc[r] * __expf(Gi - gm[r]) : 0.f;
                lds_st(lds, P_A + i * A_ROW + 4 * m0, make_float4(a[0], a[1], a[2], a[3]));
            }
        }
        __syncthreads();

        // T = (I + A)^-1 in 16 x 16 blocks. The diagonal blocks first, one per
        // wave: row r of T_ww solves (I + A_ww)^T y = e_r by right-looking back
        // substitution (once y_j is final it leaves -A[j][m] y_j in every y_m,
        // m < j; 15 dependent steps).
        if (l < 16) {
            float y[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) y[m] = m == l ? 1.f : 0.f;
#pragma unroll
            for (int j = 15; j >= 1; --j) {
#pragma unroll
                for (int mq = 0; mq < j; mq += 4) {
                    const float4 a = lds_ld<float4>(lds, P_A + (16 * w + j) * A_ROW + 4 * (16 * w + mq));
                    if (mq + 0 < j) y[mq + 0] = fmaf(-a.x, y[j], y[mq + 0]);
                    if (mq + 1 < j) y[mq + 1] = fmaf(-a.y, y[j], y[mq + 1]);
                    if (mq + 2 < j) y[mq + 2] = fmaf(-a.z, y[j], y[mq + 2]);
                    if (mq + 3 < j) y[mq + 3] = fmaf(-a.w, y[j], y[mq + 3]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                lds_st(lds, tb_off(w, w) + l * TB_ROW + 16 * q,
                       make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]));
        }
        __syncthreads();
        // Then block row by block row: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,
        // wave J taking column block J (waves J >= I wait at this level). Each
        // 16 x 16 x 16 product is four fp32 16 x 16 x 4 MFMAs: lane l supplies
        // L[l % 16][k] and R[k][l % 16] and receives D[4 (l / 16) + v][l % 16]
        // in element v, with k = 4 k4 + l / 16 in MFMA k4 of the first product,
        // and k = 4 (l / 16) + k4 in the second, whose R is then X =
        // sum_K A_IK T_KJ as the first left it in the lane.
        {
            const int lr = l & 15;
            const int lk = l >> 4;
#pragma unroll
            for (int I = 1; I < 4; ++I) {
                if (w < I) {
                    const int J = w;
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
                    for (int K = J; K < I; ++K)
#pragma unroll
                        for (int k4 = 0; k4 < 4; ++k4) {
                            const float a = lds_ld<float>(lds, P_A + (16 * I + lr) * A_ROW + 64 * K + 4 * (4 * k4 + lk));
                            const float b = lds_ld<float>(lds, tb_off(K, J) + (4 * k4 + lk) * TB_ROW + 4 * lr);
                            x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
                        }
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        const float a = lds_ld<float>(lds, tb_off(I, I) + lr * TB_ROW + 4 * (4 * lk + k4));
                        t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x[k4], t, 0, 0, 0);
                    }
#pragma unroll
                    for (int v = 0; v < 4; ++v) lds_st(lds, tb_off(I, J) + (4 * lk + v) * TB_ROW + 4 * lr, -t[v]);
                }
                __syncthreads();
            }
        }

        // T'[c][m] = T[c][m] beta_m exp(G_m) and T''[c][m] = T[c][m] beta_m, each
        // as a bf16 high part and the bf16 rounding of the rest: wave w forms
        // columns 16w .. 16w + 15 (block column w) of every row c = l.
        {
            const int I = l >> 4;
            const int r = l & 15;
            const bool ok = w <= I;
            float y[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = lds_ld<float4>(lds, (ok ? tb_off(I, w) : 0) + r * TB_ROW + 16 * q);
                y[4 * q + 0] = ok ? v.x : 0.f;
                y[4 * q + 1] = ok ? v.y : 0.f;
                y[4 * q + 2] = ok ? v.z : 0.f;
                y[4 * q + 3] = ok ? v.w : 0.f;
            }
            __syncthreads();  // every block is read before the T' parts overwrite them
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int q = 2 * w + q2;  // columns 8q .. 8q + 7
                const float4 E0 = lds_ld<float4>(lds, P_E + 32 * q);
                const float4 E1 = lds_ld<float4>(lds, P_E + 32 * q + 16);
                const float4 B0 = lds_ld<float4>(lds, P_B + 32 * q);
                const float4 B1 = lds_ld<float4>(lds, P_B + 32 * q + 16);
                const float eq[8] = {E0.x, E0.y, E0.z, E0.w, E1.x, E1.y, E1.z, E1.w};
                const float bq[8] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
                bf16x8 ph, pl, qh, ql;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float tq = y[8 * q2 + e] * bq[e];
                    const float tp = tq * eq[e];
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
        // token-major), and U = T'' V for value columns [32w, 32w + 32) (fp32, in
        // the pieces of slice w). Rows past the chunk's end come out zero.
        const buf_t rt = buf_rsrc(tile_at(p, s, h), n > 0 ? TILE_BYTES : 0);
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
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const u32x2 pw = {pack_f32(aw[4 * g4], aw[4 * g4 + 1]), pack_f32(aw[4 * g4 + 2], aw[4 * g4 + 3])};
                buf_st8(rt, 2 * (i * D + 32 * w + 8 * g4 + 4 * lh), pw);
                const u32x4 pu = {__float_as_uint(au[4 * g4]), __float_as_uint(au[4 * g4 + 1]),
                                  __float_as_uint(au[4 * g4 + 2]), __float_as_uint(au[4 * g4 + 3])};
                buf_st16(rt, T_U + 16 * ((w * 8 + 4 * nt + g4) * 64 + l), pu);
            }
        }
        __syncthreads();  // LDS is free for the next item
    }
}

// ---- gdn_chain_kernel: one workgroup per (sequence, head, block of 16 value
// columns); a ring of H_RING chunk buffers in LDS (bytes).
constexpr int H_COLS = 16;            // value columns per chain workgroup
constexpr int H_NB = D / H_COLS;      // column blocks per head
constexpr int HB_W = 0;               // W rows [64][256 B], swizzled as row_off
constexpr int HB_K = 16384;           // k rows [64][256 B], swizzled as row_off
constexpr int HB_U = 32768;           // this block's U: [token tile 4][64 lanes] x 16 B
constexpr int HB_G = 36864;           // g[64] fp32 (rows past the chunk's end: the last row's)
constexpr int H_BUF = HB_G + 256;
constexpr int H_RING = 4;             // chunk j + 3 loads while chunk j computes
// Operand stages, each in the order of the output kernel's operand images:
// piece (op, lh, c) of 16 bytes at ((2 op + lh) 16 + c) 16 holds elements
// 16 op + 4 lh + {0..3} and 16 op + 8 + 4 lh + {0..3} (keys or tokens) of
// the block's column c.
constexpr int H_SS = H_RING * H_BUF;  // the chunk's start state, bf16: 8 ops
constexpr int H_SN = H_SS + 4096;     // new_v, bf16: 4 ops
constexpr int H_XH = H_SN + 2048;     // exp(G_last - G) new_v, bf16 high part: 4 ops
constexpr int H_XL = H_XH + 2048;     // low part
constexpr int H_E = H_XL + 2048;      // exp(G_last - G)[64], one copy per compute wave
constexpr int H_CW = 2;               // compute waves
constexpr int H_BYTES = H_E + H_CW * 256;
static_assert(H_BYTES <= kLdsPerCU, "the chain workgroup must fit one CU's LDS");
constexpr int H_MOVERS = 4;           // waves that move data (after the compute waves)
constexpr int H_THREADS = 64 * (H_CW + H_MOVERS);
// Mover roles: every mover takes 16 / H_MOVERS of the W and of the k pieces;
// movers 0..3 one U token tile each; H_SMOV.. H_SMOV + 3 one quarter of the
// state image each; movers 0 and 1 half of the new_v image each; H_GMOV g.
constexpr int H_WK = 16 / H_MOVERS;
constexpr int H_SMOV = H_MOVERS == 8 ? 4 : 0;
constexpr int H_GMOV = H_MOVERS == 8 ? 4 : 0;

__device__ __forceinline__ int stage_off(int op, int lh, int c) { return ((2 * op + lh) * 16 + c) * 16; }

// Byte offset, inside the 8 KiB image slice of output wave cb / 2, of piece
// (op, lh, c) of column block cb: the output kernel's lane 32 lh + 16 (cb % 2)
// + c of operand op.
__device__ __forceinline__ int image_off(int cb, int op, int lh, int c) {
    return (op * 64 + lh * 32 + 16 * (cb & 1) + c) * 16;
}

// A sequence's chunks are consecutive tokens: its start and length come from
// its first and last table rows, read once, so the chunk loop itself reads no
// table entries (and the compiler adds no waits for them). nseg is at least 1
// for a valid table (an empty sequence has one empty row); offsets that break
// the rules can leave 0, and then no row is read.
struct ChainSeq {
    int first, nch, len;
    int64_t tok0;
};
__device__ __forceinline__ ChainSeq chain_seq(const GdnParams &p, int seq) {
    const SeqEntry sq = seq_at(p.c, seq);
    ChainSeq c{sq.first, sq.nseg, 0, 0};
    if (c.nch > 0) {
        c.tok0 = seg_at(p.c, sq.first).tok0;
        c.len = (c.nch - 1) * kChunk + max(seg_at(p.c, sq.first + c.nch - 1).len, 0);
    }
    return c;
}

// The chain workgroup has H_CW + H_MOVERS waves. Waves 0 .. H_CW - 1 hold
// the state and compute; the mover waves move every byte between HBM and LDS: chunk
// j + 3's W rows, k rows, U pieces and g into the ring by direct global ->
// LDS loads, and chunk j's state and new_v images from the LDS stages to the
// workspace, each mover an equal share. A wave is held at each load it issues
// while the memory path takes it (one wave moves about 20 bytes per ns this
// way), so the compute waves issue none and the movers split the bytes.
//
// vmcnt counts every operation a wave issues and they complete in issue
// order, so a chunk's loads are done once at most the operations issued
// after its last load remain outstanding; each mover keeps that count.
__device__ __forceinline__ void chain_mover(const GdnParams &p, int seq, int h, int cb, int mv, char *lds) {
    static_assert(H_RING == 4, "the mover keeps the counts of three chunks in flight");
    static_assert(H_MOVERS == 4 || H_MOVERS == 8, "the mover roles are laid out for four or eight movers");
    const int H = p.c.H;
    const ChainSeq c = chain_seq(p, seq);
    const int l = threadIdx.x & 63;
    const int m16 = l & 15;
    const int64_t row_bytes = (int64_t)H * D * 2;
    // This block's U pieces and state image share the bytes of its half of
    // the 8 KiB image slice of output wave cb / 2 (see gdn_prep_kernel).
    const int slice = T_U + (cb >> 1) * 8192;
    int issued = 0;  // vector-memory operations this wave has issued

    auto issue_w = [&](int j) {  // g and W rows
        const int n = min(kChunk, c.len - kChunk * j);
        const int64_t t0 = c.tok0 + (int64_t)kChunk * j;
        const char *buf = lds + (j % H_RING) * H_BUF;
        const char *tile = tile_at(p, c.first + j, h);
        if (mv == H_GMOV) {
            gll4(p.c.g + (t0 + min(l, n - 1)) * H + h, buf + HB_G);
            ++issued;
        }
#pragma unroll
        for (int i = H_WK * mv; i < H_WK * mv + H_WK; ++i) {
            const int r = 4 * i + (l >> 4);
            gll16(tile + r * 256 + ((m16 ^ (r & 15)) << 4), buf + HB_W + 1024 * i);
        }
        issued += H_WK;
    };
    auto issue_k = [&](int j) {  // k rows; rows past the chunk's end repeat its last row
        const int n = min(kChunk, c.len - kChunk * j);
        const int64_t t0 = c.tok0 + (int64_t)kChunk * j;
        const char *buf = lds + (j % H_RING) * H_BUF;
        const char *kb = static_cast<const char *>(p.c.k) + (t0 * H + h) * (D * 2);
#pragma unroll
        for (int i = H_WK * mv; i < H_WK * mv + H_WK; ++i) {
            const int r = 4 * i + (l >> 4);
            gll16(kb + min(r, n - 1) * row_bytes + ((m16 ^ (r & 15)) << 4), buf + HB_K + 1024 * i);
        }
        issued += H_WK;
    };
    auto issue_u = [&](int j) {
        // Token tile mv: lane l holds tokens 16 mv + 4 (l / 16) .. + 3 of
        // column l % 16, the piece (op, lh) = (2 mv + l / 32, (l / 16) % 2).
        if (mv >= 4) return;
        const char *buf = lds + (j % H_RING) * H_BUF;
        const int rho = 4 * mv + (l >> 4);
        // Non-temporal: each U piece is read once, by this workgroup.
        gll16_nt(tile_at(p, c.first + j, h) + slice + image_off(cb, rho >> 1, rho & 1, m16),
                 buf + HB_U + 1024 * mv);
        ++issued;
    };

    if (c.len <= 0) return;
    // issued-counts after the last load of chunks j, j + 1 and j + 2
    int mark[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if (i < c.nch) {
            issue_w(i);
            issue_k(i);
            issue_u(i);
        }
        mark[i] = issued;
    }

    // This mover's pieces of the stages: state piece 64 (mv - H_SMOV) + l,
    // new_v piece 64 mv + l for movers 0 and 1.
    const int sm = mv - H_SMOV;
    const bool s_copy = sm >= 0 && sm < 4;
    const int sp = 64 * sm + l;
    const int s_img = image_off(cb, sp >> 5, (sp >> 4) & 1, sp & 15);
    const int np = 64 * mv + l;
    const int n_img = ((cb >> 1) * 4 * 64) * 16 + image_off(cb, np >> 5, (np >> 4) & 1, np & 15);

    for (int j = 0; j < c.nch; ++j) {
        wait_vm_n(__builtin_amdgcn_readfirstlane(min(issued - mark[0], 63)));
        __syncthreads();  // chunk j is in LDS; chunk j - 1's buffer is free
        const int jn = j + 3;
        const bool more = jn < c.nch;
        if (more) issue_w(jn);
        __syncthreads();  // the state operands are staged
        if (s_copy) {
            // Non-temporal (as the new_v image below): the images are read only
            // by the output kernel, and kept out of L2 they leave it to the W
            // and k rows the head's other column blocks still read.
            const bf16x8 x = lds_ld<bf16x8>(lds, H_SS + 16 * sp);
            __builtin_nontemporal_store(x, reinterpret_cast<bf16x8 *>(tile_at(p, c.first + j, h) + slice + s_img));
            ++issued;
        }
        if (more) issue_k(jn);
        __syncthreads();  // new_v is staged
        if (more) issue_u(jn);
        const int mark2 = issued;
        if (mv < 2) {
            const bf16x8 x = lds_ld<bf16x8>(lds, H_SN + 16 * np);
            __builtin_nontemporal_store(
                x, reinterpret_cast<bf16x8 *>(p.nvimg + ((int64_t)(c.first + j) * H + h) * NV_BYTES + n_img));
            ++issued;
        }
        mark[0] = mark[1];
        mark[1] = mark[2];
        mark[2] = mark2;
    }
}

// The state recurrence of one (sequence, head, block of 16 value columns)
// per workgroup: W and k of a chunk are read by the eight blocks of a head
// (the eight workgroups sit on one XCD and share its L2); U, the state and
// the images are the block's own. Compute wave a (of H_CW) holds key tiles
// KT a .. KT a + KT - 1 of the block's state, KT = 8 / H_CW, as 16 x 16
// tiles (tile t: lane l holds key 16t + 4(l/16) + v, column l % 16, in
// element v), and forms new_v for token tiles TT a .. TT a + TT - 1,
// TT = 4 / H_CW (16 tokens each).
//
// Per chunk, on 16 x 16 x 32 bf16 MFMAs: the compute waves stage their state
// as bf16 operands, so each forms new_v = U - W S for its token half over all
// key rows; then they stage exp(G_last - G) new_v as bf16 high and low parts,
// so each updates its key rows with all 64 tokens (K^T from the k rows
// through the transposing read). Inside one MFMA the order of the 32 k values
// is free as long as both operands follow it; here it is the order of the
// stage pieces, so the stages are at once the operands and the images.
// The work of compute wave WA (a compile-time index, so that every register
// array is indexed by constants); all waves pass the same barriers in the
// same order.
template <int WA>
__device__ __forceinline__ void chain_wave(const GdnParams &p, int seq, int h, int cb, char *lds) {
    static_assert(H_CW == 2 || H_CW == 4, "two or four compute waves");
    constexpr int wa = WA;
    constexpr int KT = 8 / H_CW;  // key tiles of this wave
    constexpr int TT = 4 / H_CW;  // token tiles of this wave
    const int H = p.c.H;
    const ChainSeq c = chain_seq(p, seq);
    const int l = threadIdx.x & 63;
    const int lc = l & 15;   // column (state, new_v) or row (W, K^T) of a 16 x 16 tile
    const int g = l >> 4;    // lane group
    const int64_t sl = (int64_t)D * D;
    const int col = H_COLS * cb + lc;

    f32x4 S[KT];
    {
        const float *src = p.c.s0 ? p.c.s0 + ((int64_t)seq * H + h) * sl : nullptr;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                S[t][v] = src ? src[(16 * (KT * wa + t) + 4 * g + v) * D + col] : 0.f;
    }

    // The k values lane group g supplies in step ks of 32: 32 ks + o(g) + {0..3}
    // and + 8 + {0..3}, o(g) = 16 (g / 2) + 4 (g % 2): stage piece
    // (2 ks + g / 2, g % 2). Lane-constant parts of the transposing reads of
    // K^T (key tile t, the two 4-token halves).
    const int og = 16 * (g >> 1) + 4 * (g & 1);
    int trk[KT][2];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) trk[t][hf] = tr_src(og + 8 * hf, 16 * (KT * wa + t), lc);

    const int nch = c.len > 0 ? c.nch : 0;
    for (int j = 0; j < nch; ++j) {
        __syncthreads();  // chunk j is in LDS
        const char *buf = lds + (j % H_RING) * H_BUF;
        const int n = min(kChunk, c.len - kChunk * j);
        const float G = wave_prefix_sum(l < n ? lds_ld<float>(buf, HB_G + 4 * l) : 0.f);
        const float Gl = lane_value(G, 63);
        // exp(G_last - G) of token l, once per token
        lds_st(lds, H_E + 256 * wa + 4 * l, __expf(Gl - G));

        // This wave's state tiles as bf16 stage pieces: key tile KT wa + t,
        // lane group g -> piece (KT wa + t, g % 2), half g / 2.
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const bf16x4 x = {(__bf16)S[t][0], (__bf16)S[t][1], (__bf16)S[t][2], (__bf16)S[t][3]};
            lds_st(lds, H_SS + stage_off(KT * wa + t, g & 1, lc) + 8 * (g >> 1), x);
        }
        __syncthreads();  // the whole state is staged

        // new_v = U - W S for this wave's token tiles over all key rows.
        f32x4 acc[TT] = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 sb = lds_ld<bf16x8>(lds, H_SS + stage_off(2 * ks + (g >> 1), g & 1, lc));
            const int c1 = 4 * ks + 2 * (g >> 1);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const int i = 16 * (TT * wa + tt) + lc;
                const bf16x4 x0 = lds_ld<bf16x4>(buf, HB_W + row_off(i, c1) + 8 * (g & 1));
                const bf16x4 x1 = lds_ld<bf16x4>(buf, HB_W + row_off(i, c1 + 1) + 8 * (g & 1));
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat4(x0, x1), sb, acc[tt], 0, 0, 0);
            }
        }
        // Its bf16 image for the output kernel, and exp(G_last - G) new_v as
        // high and low bf16 parts for every wave's update.
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int q = TT * wa + tt;  // token tile
            const float4 u = lds_ld<float4>(buf, HB_U + 1024 * q + 16 * l);
            const float4 e = lds_ld<float4>(lds, H_E + 256 * wa + 4 * (16 * q + 4 * g));
            const float uq[4] = {u.x, u.y, u.z, u.w};
            const float eq[4] = {e.x, e.y, e.z, e.w};
            bf16x4 nvo, xh, xl;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float nv = uq[v] - acc[tt][v];
                const float x = nv * eq[v];
                nvo[v] = (__bf16)nv;
                xh[v] = (__bf16)x;
                xl[v] = (__bf16)(x - (float)xh[v]);
            }
            const int so = stage_off(q, g & 1, lc) + 8 * (g >> 1);
            lds_st(lds, H_SN + so, nvo);
            lds_st(lds, H_XH + so, xh);
            lds_st(lds, H_XL + so, xl);
        }
        __syncthreads();  // every token tile of new_v is staged

        if (j + 1 < nch || p.c.sfin) {
            const float a = __expf(Gl);
#pragma unroll
            for (int t = 0; t < KT; ++t) S[t] *= a;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int so = stage_off(2 * ks + (g >> 1), g & 1, lc);
                const bf16x8 xh = lds_ld<bf16x8>(lds, H_XH + so);
                const bf16x8 xl = lds_ld<bf16x8>(lds, H_XL + so);
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    const bf16x8 kt = cat4(lds_tr(buf, HB_K + 8192 * ks + trk[t][0]),
                                           lds_tr(buf, HB_K + 8192 * ks + trk[t][1]));
                    S[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, xh, S[t], 0, 0, 0);
                    S[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, xl, S[t], 0, 0, 0);
                }
            }
        }
    }

    if (p.c.sfin) {
        float *dst = p.c.sfin + ((int64_t)seq * H + h) * sl;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) dst[(16 * (KT * wa + t) + 4 * g + v) * D + col] = S[t][v];
    }
}

__global__ __launch_bounds__(H_THREADS) void gdn_chain_kernel(GdnParams p) {
    int unit, cb;
    xcd_unit_map(blockIdx.x, H_NB, unit, cb);
    const int seq = unit / p.c.H;
    const int h = unit - seq * p.c.H;
    if (seq >= p.c.N) return;
    __shared__ __attribute__((aligned(16))) char lds[H_BYTES];
    const int w = threadIdx.x >> 6;
    if (w >= H_CW) chain_mover(p, seq, h, cb, w - H_CW, lds);
    else if (w == 0) chain_wave<0>(p, seq, h, cb, lds);
    else if (w == 1) chain_wave<1>(p, seq, h, cb, lds);
    else if (H_CW > 2 && w == 2) chain_wave<2 % H_CW>(p, seq, h, cb, lds);
    else if (H_CW > 3) chain_wave<3 % H_CW>(p, seq, h, cb, lds);
}

// ---- gdn_output_kernel LDS map (bytes).
constexpr int O_Q = 0;       // Q rows [64][256 B]
constexpr int O_K = 16384;   // K rows [64][256 B]; later the O staging rows
constexpr int O_A = 32768;   // scores A[64 i][128 B], bf16 high part
constexpr int O_AL = 40960;  // low part
constexpr int O_G = 49152;   // G[64] fp32
constexpr int O_BYTES = O_G + 256;
static_assert(3 * O_BYTES <= kLdsPerCU, "three output workgroups must fit one CU's LDS");

// One (chunk, head) per workgroup, all chunks at once:
// O = scale ((Q * exp(G)) S + lower(Q K^T * Gamma) new_v), with S (the state
// the chunk starts from) and new_v taken in bf16 from the chain kernel's
// images, and the scores split into bf16 high and low parts (the product of
// rounded scores and rounded new_v is the largest part of the bf16 error).
// Wave w computes value columns [32w, 32w + 32) of O.
__global__ __launch_bounds__(NT) void gdn_output_kernel(GdnParams p) {
    const int H = p.c.H;
    const int s = blockIdx.x / H;
    const int h = blockIdx.x - s * H;
    if (s >= p.c.nseg_max) return;
    const SegEntry se = seg_at(p.c, s);
    if (se.len <= 0) return;
    const int n = se.len;
    __shared__ __attribute__((aligned(16))) char lds[O_BYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int l = tid & 63;
    const int ln = l & 31;
    const int lh = l >> 5;
    const int cidx = tid & 15;
    const int prb = (tid >> 4) & 15;

    const int64_t base = (se.tok0 * H + h) * D;
    const uint16_t *qg = static_cast<const uint16_t *>(p.c.q) + base;
    const uint16_t *kg = static_cast<const uint16_t *>(p.c.k) + base;
    const int64_t rs = (int64_t)H * D;
    u32x4 qr[2][2], kr[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * (prb + 16 * it) + rr;
            const bool ok = r < n;
            qr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(qg + r * rs + 8 * cidx) : u32x4{0, 0, 0, 0};
            kr[it][rr] = ok ? *reinterpret_cast<const u32x4 *>(kg + r * rs + 8 * cidx) : u32x4{0, 0, 0, 0};
        }
    const float gv = l < n ? p.c.g[(se.tok0 + l) * H + h] : 0.f;
    const char *img = tile_at(p, s, h) + IMG_S;
    const char *nimg = p.nvimg + ((int64_t)s * H + h) * NV_BYTES;
    // Non-temporal: each image is read once, here.
    bf16x8 sb[8], nvop[4];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        sb[k] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(img + ((w * 8 + k) * 64 + l) * 16));
#pragma unroll
    for (int k = 0; k < 4; ++k)
        nvop[k] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(nimg + ((w * 4 + k) * 64 + l) * 16));

    const float G = wave_prefix_sum(gv);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * (prb + 16 * it) + rr;
            lds_st(lds, O_Q + row_off(r, cidx), qr[it][rr]);
            lds_st(lds, O_K + row_off(r, cidx), kr[it][rr]);
        }
    if (w == 0) lds_st(lds, O_G + 4 * l, G);
    __syncthreads();

    // Scores: wave 0 -> (j 0-31, i 0-31), 1 -> (j 0-31, i 32-63), 2 -> (j 32-63, i 32-63).
    if (w < 3) {
        const int jb = w == 2 ? 1 : 0;
        const int ib = w == 0 ? 0 : 1;
        f32x16 acc = {};
        const int jj = 32 * jb + ln;
        const int i = 32 * ib + ln;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const bf16x8 a = lds_ld<bf16x8>(lds, O_K + row_off(jj, 2 * st + lh));
            const bf16x8 bq = lds_ld<bf16x8>(lds, O_Q + row_off(i, 2 * st + lh));
            acc = mfma(a, bq, acc);
        }
        const float Gi = lds_ld<float>(lds, O_G + 4 * i);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int jr = 32 * jb + 8 * g4 + 4 * lh;
            const float4 Gj = lds_ld<float4>(lds, O_G + 4 * jr);
            const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
            float val[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                val[r] = (jr + r <= i) ? p.c.scale * __expf(Gi - gj[r]) * acc[4 * g4 + r] : 0.f;
            // bf16 high part and the bf16 rounding of the rest
            float lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) lo[r] = val[r] - round_bf16(val[r]);
            const u32x2 pk = {pack_f32(val[0], val[1]), pack_f32(val[2], val[3])};
            const u32x2 pl = {pack_f32(lo[0], lo[1]), pack_f32(lo[2], lo[3])};
            lds_st(lds, O_A + tr_off(i, 4 * jb + g4) + 8 * lh, pk);
            lds_st(lds, O_AL + tr_off(i, 4 * jb + g4) + 8 * lh, pl);
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
                const bf16x4 x0 = lds_ld<bf16x4>(lds, O_Q + row_off(i, c) + 8 * lh);
                const bf16x4 x1 = lds_ld<bf16x4>(lds, O_Q + row_off(i, c + 1) + 8 * lh);
                acc = mfma(sb[2 * b + s2], cat4(x0, x1), acc);
            }
        const float f = p.c.scale * __expf(lds_ld<float>(lds, O_G + 4 * i));
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] *= f;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (nt == 0 && st >= 2) break;
            const bf16x4 y0 = lds_ld<bf16x4>(lds, O_A + tr_off(i, 2 * st) + 8 * lh);
            const bf16x4 y1 = lds_ld<bf16x4>(lds, O_A + tr_off(i, 2 * st + 1) + 8 * lh);
            const bf16x4 z0 = lds_ld<bf16x4>(lds, O_AL + tr_off(i, 2 * st) + 8 * lh);
            const bf16x4 z1 = lds_ld<bf16x4>(lds, O_AL + tr_off(i, 2 * st + 1) + 8 * lh);
            acc = mfma(nvop[st], cat4(y0, y1), acc);
            acc = mfma(nvop[st], cat4(z0, z1), acc);
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 pk = {pack_f32(acc[4 * g4], acc[4 * g4 + 1]),
                              pack_f32(acc[4 * g4 + 2], acc[4 * g4 + 3])};
            lds_st(lds, O_K + row_off(i, 4 * w + g4) + 8 * lh, pk);
        }
    }
    __syncthreads();  // O staging rows complete
    uint16_t *og = static_cast<uint16_t *>(p.c.out) + base;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * (prb + 16 * it) + rr;
            if (r < n)  // non-temporal: nothing in the call reads the output again
                __builtin_nontemporal_store(lds_ld<u32x4>(lds, O_K + row_off(r, cidx)),
                                            reinterpret_cast<u32x4 *>(og + r * rs + 8 * cidx));
        }
}

}  // namespace

hipError_t launch_gdn_chunk(const GdnParams &p, hipStream_t st) {
    if (p.c.N == 0) return hipSuccess;
    const dim3 chunks((unsigned)((int64_t)p.c.nseg_max * p.c.H));
    if (p.c.nseg_max > 0) {
        // Two workgroups fit on a CU (72 KiB of LDS each).
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        const int64_t nitems = (int64_t)p.c.nseg_max * p.c.H;
        const unsigned wgs = (unsigned)std::min<int64_t>(nitems, 2 * (int64_t)cus);
        hipLaunchKernelGGL(gdn_prep_kernel, dim3(wgs), dim3(NT), 0, st, p, (int)nitems);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // H_NB column blocks per (sequence, head), the units rounded up to whole
    // groups of eight so that xcd_unit_map covers them.
    const int64_t units = ((int64_t)p.c.N * p.c.H + 7) / 8 * 8;
    hipLaunchKernelGGL(gdn_chain_kernel, dim3((unsigned)(units * H_NB)), dim3(H_THREADS), 0, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.c.nseg_max > 0) hipLaunchKernelGGL(gdn_output_kernel, chunks, dim3(NT), 0, st, p);
    return hipGetLastError();
}

}  // namespace sgla
