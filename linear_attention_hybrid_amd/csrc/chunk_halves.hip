// Chunked Simple GLA output pass over value-column halves: bf16 operands,
// fp32 accumulation, Dk = Dv = 128, chunks of 64 tokens.
//
// Per chunk with inclusive cumulative gate sums G (page "Formulas and code for
// adapting inference to GDN/KDA linear modules", section 1.2, reduced to Simple
// GLA: no delta-rule terms, new_v = v; the diagonal is included because the
// query reads the state after the token's own update, blueprint page, section
// "B2 lightning-attn (Simple GLA)"):
//
//   A   = scale * (Q K^T) * exp(G_i - G_j) for j <= i, else 0
//   O   = scale * diag(exp(G)) Q S + A V
//   S   = exp(G_last) * S + K^T (diag(exp(G_last - G)) V)
//
// One workgroup owns one output segment of one head and one half of the value
// columns (64 of 128), so a head's segment is split over two workgroups that
// share the q and k rows through their XCD's L2. It is four waves, and two
// workgroups share a compute unit, so that one's memory and LDS latency hides
// behind the other's work. Each thread loads its share of the next chunk's q
// and k rows, the half's v rows and g into registers with range-checked buffer
// loads while the current chunk is computed, and writes them into the LDS
// tiles at the top of the next iteration; rows past a ragged end read as
// zeros. Wave (cc, t) owns value columns 32cc .. 32cc+31 of the half; for the
// output it takes token half t (tokens 32t .. 32t+31), and of the fp32 state
// it holds key rows 64t .. 64t+63 in MFMA accumulators. Each wave forms Q S
// over its own 64 key rows for all 64 tokens, and the two waves of one column
// block trade the fp32 partial sums of each other's tokens through LDS.
//
// The products are 32x32x16 bf16 MFMAs, each written so that its result is
// already in the register layout the next consumes (see mfma_tile.h): the
// state accumulators convert to the A operand of S^T Q^T, as a bf16 pair
// hi + lo (two MFMAs), so that the state keeps about 16 bits in the output:
// one bf16 rounding of a large, slowly decaying state would cost the outputs
// 2^-9 of their size. A^T = K Q^T leaves
// each lane one query column, stored as A[i][j] rows for the B operand of
// V^T A^T. K^T and V^T operands come from the row-major tiles through the
// transposing LDS read, and the decay exp(G_last - G) scales the V operand of
// the update (one bf16 rounding, as scaling K would be). Output rows go
// through an LDS staging tile, so each row's 128 bytes are stored as one line.
//
// The start state of a segment is the initial state, or, when the sequence
// spans several output segments, the initial state and the states of the
// sub-segments before it (from the state pass), combined at the start of the
// workgroup: this path needs no scan kernel.
#include "mfma_tile.h"

namespace sgla {

namespace {

constexpr int D = 128;
constexpr int NTH = 256;              // four waves
// LDS map (bytes); two workgroups share a compute unit.
constexpr int L_Q = 0;                // Q rows [64][256 B], swizzled as qk_off
constexpr int L_K = 16384;            // K rows, same layout
constexpr int L_V = 32768;            // the half's V rows [64][128 B], swizzled as v_off
constexpr int L_A = 40960;            // scores A[64 i][128 B] bf16, swizzled as tr_off
constexpr int L_SX = L_A + 8192;      // fp32 partials of Q S [block cc 2][token half 2][4][lane 64] x 16 B
constexpr int L_O = L_SX + 16384;     // output staging [64 rows][128 B], swizzled as o_off; first the update's V operand halves passed between partner waves
constexpr int L_F = L_O + 8192;       // per wave: G[64] and exp(G_last - G)[64], fp32
constexpr int L_BYTES = L_F + 4 * 512;
static_assert(2 * L_BYTES <= kLdsPerCU, "two workgroups must fit one compute unit's LDS");

// Q and K tiles (64 rows of 256 bytes): 16-byte chunk c of row r sits at
// chunk c ^ qk_sw(r). Sixteen consecutive rows then put one chunk in 16
// different bank groups, so the 16-byte operand reads of the scores and of
// Q S, one row per lane, are free of bank conflicts, and the four rows of a
// transposing read put an aligned group of four chunks in 16 different bank
// groups (the K^T reads of the update).
__device__ __forceinline__ int qk_sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int qk_off(int r, int c) { return r * 256 + ((c ^ qk_sw(r)) << 4); }
// Transposing-read address (rows r0 .. r0+3, columns c0 .. c0+15; r0 a
// multiple of 4, c0 a multiple of 16) for lane m of a 16-lane group. Lane m
// names 4-column piece kPiece[m % 4], so lane i of the group receives column
// c0 + sigma(i), sigma = (0-3, 8-11, 4-7, 12-15). The update's K^T operand
// then leaves state row rho of each 32-row block holding key dim sigma(rho)
// of it (sigma applied to each 16-row half), and the eight k values a lane
// gives Q S (state rows 4lh + 0..3 and 8 + 4lh + 0..3 of a 16-row group)
// are the eight consecutive dims 8lh .. 8lh + 7: one 16-byte Q read.
__device__ __forceinline__ int qk_tr_src(int r0, int c0, int m) {
    const int r = r0 + (m >> 2);
    const int pc = ((m & 1) << 1) | ((m >> 1) & 1);  // kPiece = (0, 2, 1, 3)
    return qk_off(r, (c0 >> 3) + (pc >> 1)) + 8 * (pc & 1);
}
// Key dim, within the state block of key rows 32 b .. 32 b + 31, of the state
// value a lane (half lh of the wave) holds in accumulator element v.
__device__ __forceinline__ int state_dim(int v, int lh) {
    return 16 * (v >> 3) + 4 * ((v >> 2) & 1) + 8 * lh + (v & 3);
}
__device__ __forceinline__ u32x4 swap_halves(u32x4 x) { return u32x4{x[2], x[3], x[0], x[1]}; }

// V half tile: 16-byte piece p of row r. Rows r and r + 2 differ in bit 2 of
// the swizzle, so the four rows of one transposing read fill 16 different
// bank groups.
__device__ __forceinline__ int v_off(int r, int p) { return r * 128 + ((p ^ (((r >> 1) & 1) << 2)) << 4); }
// Byte offset of the 8 bytes lane m of a 16-lane group names for the
// transposing read of rows r0 .. r0+3, columns c0 .. c0+15 of the V tile
// (r0 a multiple of 4, c0 a multiple of 16).
__device__ __forceinline__ int vtr_src(int r0, int c0, int m) {
    return v_off(r0 + (m >> 2), (c0 >> 3) + ((m & 3) >> 1)) + 8 * (m & 1);
}
// Output staging tile (64 rows of 128 bytes): piece p of row r at piece
// p ^ ((r >> 1) & 7), halves traded in rows with bit 4 set, so that the
// 8-byte writes of 32 consecutive rows fill all banks once.
__device__ __forceinline__ int o_off(int r, int p) { return r * 128 + ((p ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int o_half(int r, int hf) { return 8 * (hf ^ ((r >> 4) & 1)); }
__device__ __forceinline__ int sx_off(int cc, int ib, int v4, int l) {
    return L_SX + (((cc * 2 + ib) * 4 + v4) * 64 + l) * 16;
}

// Output segment s of the call (without a table as seg_at).
__device__ __forceinline__ SegEntry oseg_at(const HalvesParams &hp, int s) {
    if (hp.osegs) return hp.osegs[s];
    if (hp.c.cu) return seg_from_cu(hp.c.cu, s, hp.c.T);
    SegEntry e;
    const int n = s / hp.onps;
    const int j = s - n * hp.onps;
    e.seq = n;
    e.p = j;
    e.nseg = hp.onps;
    e.tok0 = (int64_t)n * hp.c.T + (int64_t)j * hp.oseg_len;
    const int rem = hp.c.T - j * hp.oseg_len;
    e.len = rem < hp.oseg_len ? rem : hp.oseg_len;
    e.pad0 = 0;
    e.pad1 = 0;
    return e;
}

template <int TH>
__device__ void halves_wave(const HalvesParams &hp, const SegEntry &se, int h, int half, char *lds) {
    const ChunkParams &p = hp.c;
    const int H = p.H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l = tid & 63;
    const int cc = w >> 1;   // 32-column block of the half
    constexpr int t = TH;    // token half of the output, key-row half of the state
    const int lh = l >> 5;
    const int ln = l & 31;
    const int m16 = l & 15;
    const int gi = l >> 4;
    const int col = half * 64 + 32 * cc + ln;  // this lane's value column
    const int len = se.len;
    const int nch = (len + 63) >> 6;
    const bool last = se.p == se.nseg - 1;
    const int64_t sl = (int64_t)D * D;
    const uint16_t *__restrict__ qg = static_cast<const uint16_t *>(p.q);
    const uint16_t *__restrict__ kg = static_cast<const uint16_t *>(p.k);
    const uint16_t *__restrict__ vg = static_cast<const uint16_t *>(p.v);
    char *og = static_cast<char *>(p.out);

    // This thread's share of a chunk: q and k pieces (tid & 15) of rows
    // (tid >> 4) + 16 i, v piece (tid & 7) of rows (tid >> 3) + 32 i, and for
    // the first wave g of token l; a per-chunk buffer resource whose range
    // ends at the chunk's last row, so rows past a ragged end read as zeros.
    u32x4 qr[4], kr[4], vr[2];
    float gr = 0.f;
    // Bytes from a chunk's first row to the end of its row n - 1 (< 2^31
    // for H <= 65536); 0 for a chunk past the end (n <= 0), whose loads then
    // read zeros and whose stores are dropped. The loop issues the same loads
    // and stores on every path (a chunk past the end, every wave's g), so the
    // compiler's waits count exactly and the output stores stay in flight.
    auto rows_bytes = [&](int n) -> int { return n > 0 ? (n - 1) * H * (D * 2) + D * 2 : 0; };
    auto issue = [&](int c) {
        int tv = tid;
        asm volatile("" : "+v"(tv));
        const int n = min(64, len - 64 * c);
        const int64_t t0 = se.tok0 + 64 * (int64_t)c;
        const int64_t base = (t0 * H + h) * D;
        const int nb = rows_bytes(n);
        const buf_t rq = buf_rsrc(qg + base, nb);
        const buf_t rk = buf_rsrc(kg + base, nb);
        const buf_t rv = buf_rsrc(vg + base + half * 64, nb > 0 ? nb - 128 : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = (uint32_t)((tv >> 4) + 16 * i) * (uint32_t)(H * D * 2) + (tv & 15) * 16u;
            qr[i] = buf_ld16(rq, off);
            kr[i] = buf_ld16(rk, off);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t off = (uint32_t)((tv >> 3) + 32 * i) * (uint32_t)(H * D * 2) + (tv & 7) * 16u;
            vr[i] = buf_ld16(rv, off);
        }
        gr = buf_ld_f32(buf_rsrc(p.g + t0 * H + h, n > 0 ? (n - 1) * H * 4 + 4 : 0), (uint32_t)(tv & 63) * H * 4);
    };
    // Chunk c's output rows from the staging tile; with ok false (before the
    // first chunk) the same stores go out with an empty range and are dropped.
    auto store_o = [&](int c, bool ok) {
        int tv = tid;
        asm volatile("" : "+v"(tv));
        const int n = min(64, len - 64 * c);
        const int64_t t0 = se.tok0 + 64 * (int64_t)c;
        const buf_t ro = buf_rsrc(og + (t0 * H + h) * (D * 2) + half * 128, ok ? (n - 1) * H * (D * 2) + 128 : 0);
        // Bit 4 of this thread's rows is bit 1 of its wave index (tv >> 3
        // < 32), so whether the halves of its pieces trade places is the
        // same for the whole wave.
        u32x4 x[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) x[i] = lds_ld<u32x4>(lds, L_O + o_off((tv >> 3) + 32 * i, tv & 7));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (tv >> 3) + 32 * i;
            buf_st16_nt(ro, (uint32_t)r * (uint32_t)(H * D * 2) + (tv & 7) * 16u, (w & 2) ? swap_halves(x[i]) : x[i]);
        }
    };

    // The start state, key tiles 2t and 2t + 1 of this column block: the
    // initial state decayed over the sub-segments before this output
    // segment, plus each of their zero-start states (left by the state pass
    // with its total log-decay) decayed over the sub-segments after it: the
    // recurrence regrouped. The weights come from running sums of the
    // log-decays, taken from the nearest sub-segment back, so every load is
    // independent of the others. The first chunk's loads go first, so that
    // they land while the states are read; one state is in flight at a time,
    // which leaves registers for them.
    if (nch > 0) issue(0);
    f32x16 S[2] = {};
    {
        const int nj = se.nseg == 1 ? 0 : p.rsub * se.p;  // sub-segments before this segment
        const int first = nj > 0 ? seq_at(p, se.seq).first : 0;
        // This lane's 32 values of the state at `src`, all loads issued
        // before any is used: the opaque step needs every value, so the
        // compiler cannot interleave each load with its use.
        auto fetch = [&](const float *src, float (&x)[32]) {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int v = 0; v < 16; ++v) x[16 * bi + v] = src[(32 * (2 * t + bi) + state_dim(v, lh)) * D + col];
        };
        auto settle32 = [](float (&x)[32]) {
            asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                         "+v"(x[6]), "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]),
                         "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
            asm volatile("" : "+v"(x[16]), "+v"(x[17]), "+v"(x[18]), "+v"(x[19]), "+v"(x[20]), "+v"(x[21]),
                         "+v"(x[22]), "+v"(x[23]), "+v"(x[24]), "+v"(x[25]), "+v"(x[26]), "+v"(x[27]),
                         "+v"(x[28]), "+v"(x[29]), "+v"(x[30]), "+v"(x[31]));
        };
        auto add = [&](float wgt, const float (&x)[32]) {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[bi][v] = fmaf(wgt, x[16 * bi + v], S[bi][v]);
        };
        // Clamped into the buffer, so that offsets that break the documented
        // rule cannot send a read past it.
        auto slot_of = [&](int i) { return min(first + i, p.nseg_max - 1); };
        auto dstate = [&](int i) { return p.buf + ((int64_t)slot_of(i) * H + h) * sl; };
        auto lgam = [&](int i) { return p.gam[(int64_t)slot_of(i) * H + h]; };
        float tail = 0.f;  // log-decay of the sub-segments after i, up to this segment
        for (int i = nj - 1; i >= 0; --i) {
            float x0[32];
            fetch(dstate(i), x0);
            settle32(x0);
            add(__expf(tail), x0);
            tail += lgam(i);
        }
        if (p.s0) {
            float x0[32];
            fetch(p.s0 + ((int64_t)se.seq * H + h) * sl, x0);
            settle32(x0);
            add(__expf(tail), x0);
        }
    }

    char *ft = lds + L_F + 512 * w;  // this wave's G log2(e) [64], then exp(G_last - G)[64]
    const int i = 32 * t + ln;        // this lane's query row of the output
    // The scores' and rows' exponentials take base 2 with log2|scale| added
    // to the exponent: |scale| exp(G_i - G_j) = exp2(G_i log2(e) +
    // log2|scale| - G_j log2(e)); a negative scale flips the output rows.
    const float ls = __builtin_amdgcn_logf(fabsf(p.scale));
    const bool neg = p.scale < 0.f;
    const uint32_t sgn2 = neg ? 0x80008000u : 0u;  // sign bits of a bf16 pair
    for (int c = 0; c < nch; ++c) {
        const int n = min(64, len - 64 * c);
        __syncthreads();  // the previous chunk's tiles and staging are read
        store_o(c - 1, c > 0);
        {
            int tv = tid;
            asm volatile("" : "+v"(tv));
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int r = (tv >> 4) + 16 * i4;
                lds_st(lds, L_Q + qk_off(r, tv & 15), qr[i4]);
                lds_st(lds, L_K + qk_off(r, tv & 15), kr[i4]);
            }
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) lds_st(lds, L_V + v_off((tv >> 3) + 32 * i2, tv & 7), vr[i2]);
        }
        // Gate prefix sum over this wave's own copy of g, one lane per token
        // (rows past the end read as 0), and the wave's gate table, before
        // the barrier: the table is the wave's own, and its reads of the
        // previous chunk's values came first (a wave's LDS accesses complete
        // in order).
        const float G = wave_prefix_sum(gr);
        const float Gl = lane_value(G, 63);
        lds_st(ft, 4 * l, G * 1.44269504088896341f);
        lds_st(ft, 256 + 4 * l, l < n ? __expf(Gl - G) : 0.f);
        __syncthreads();  // chunk c's tiles are in LDS
        issue(c + 1);

        // O^T = S^T Q^T over this wave's key rows for both token halves;
        // the other half's partial sums go to the partner wave.
        f32x16 acc = {}, oth = {};
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                bf16x8 sh, sl;
                {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = S[bi][8 * s2 + e];
                    split_bf16x8(x, sh, sl);
                }
                const int cq = 4 * (2 * t + bi) + 2 * s2 + lh;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const int iq = 32 * ib + ln;
                    const bf16x8 bq = lds_ld<bf16x8>(lds, L_Q + qk_off(iq, cq));
                    if (ib == t) {
                        acc = mfma(sh, bq, acc);
                        acc = mfma(sl, bq, acc);
                    } else {
                        oth = mfma(sh, bq, oth);
                        oth = mfma(sl, bq, oth);
                    }
                }
            }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
            lds_st(lds, sx_off(cc, 1 - t, v4, l),
                   make_float4(oth[4 * v4], oth[4 * v4 + 1], oth[4 * v4 + 2], oth[4 * v4 + 3]));

        // Scores: wave 0 -> (keys 0-31, queries 0-31), 1 -> (0-31, 32-63),
        // 3 -> (32-63, 32-63); the fourth quadrant is masked out.
        if (w != 2) {
            const int jb = w == 3 ? 1 : 0;
            const int ib = w == 0 ? 0 : 1;
            const int j = 32 * jb + ln;
            const int iq = 32 * ib + ln;
            f32x16 sc = {};
#pragma unroll
            for (int s8 = 0; s8 < 8; ++s8) {
                const bf16x8 a = lds_ld<bf16x8>(lds, L_K + qk_off(j, 2 * s8 + lh));
                const bf16x8 bq = lds_ld<bf16x8>(lds, L_Q + qk_off(iq, 2 * s8 + lh));
                sc = mfma(a, bq, sc);
            }
            const float Gi = lds_ld<float>(ft, 4 * iq) + ls;
            // Keys past the query are cleared after packing, by a mask on
            // each bf16 of a pair: no branch, and an infinite or NaN product
            // there (exp of a positive gate sum) is cleared as well. Wave 1
            // pairs keys 0-31 with queries 32-63 and keeps every key. A
            // negative scale flips the sign bits.
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int jr = 32 * jb + 8 * g4 + 4 * lh;
                const float4 Gj = lds_ld<float4>(ft, 4 * jr);
                const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
                float val[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) val[r] = __builtin_amdgcn_exp2f(Gi - gj[r]) * sc[4 * g4 + r];
                u32x2 pk = {pack_f32(val[0], val[1]), pack_f32(val[2], val[3])};
                const int d = w == 1 ? 64 : iq - jr;  // key jr + r is kept when r <= d
                pk[0] &= (d >= 1 ? 0xffffffffu : 0u) | (d >= 0 ? 0x0000ffffu : 0u);
                pk[1] &= (d >= 3 ? 0xffffffffu : 0u) | (d >= 2 ? 0x0000ffffu : 0u);
                pk[0] ^= sgn2;
                pk[1] ^= sgn2;
                lds_st(lds, L_A + tr_off(iq, 4 * jb + g4) + 8 * lh, pk);
            }
        }

        // V^T operands (lane: value column 32cc + ln, tokens 16s + 8lh .. + 7),
        // shared by V^T A^T and the update.
        bf16x8 vop[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int c0 = 32 * cc + 16 * (gi & 1);
            vop[s4] = cat4(lds_tr(lds, L_V + vtr_src(16 * s4 + 8 * lh, c0, m16)),
                           lds_tr(lds, L_V + vtr_src(16 * s4 + 8 * lh + 4, c0, m16)));
        }
        // The update's V operand, exp(G_last - G) V: this wave forms tokens
        // 32t .. 32t+31 (s4 = 2t, 2t+1), which its partner (cc, 1-t) needs as
        // well, and hands them over in the partner's own output-staging
        // slots (rows 32(1-t) .., pieces 4cc ..), unused until the partner
        // stages its output after reading them; it takes the other two from
        // its own slots after the barrier.
        const bool upd = c + 1 < nch || (last && p.sfin);
        bf16x8 vs[4];
        if (upd) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int s4 = 2 * t + k;
                const float4 f0 = lds_ld<float4>(ft, 256 + 4 * (16 * s4 + 8 * lh));
                const float4 f1 = lds_ld<float4>(ft, 256 + 4 * (16 * s4 + 8 * lh) + 16);
                const float fe[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
                float xs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xs[e] = (float)vop[s4][e] * fe[e];
                vs[s4] = to_bf16x8(xs);
                lds_st(lds, L_O + o_off(32 * (1 - t) + ln, 4 * cc + 2 * k + lh), vs[s4]);
            }
        }
        __syncthreads();  // the scores, the partial sums and the V operand halves are staged

        // The partner's key rows, then the rows scaled by scale * exp(G_i).
        {
            const float fa = __builtin_amdgcn_exp2f(lds_ld<float>(ft, 4 * i) + ls);
            const float f = neg ? -fa : fa;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const float4 y = lds_ld<float4>(lds, sx_off(cc, t, v4, l));
                acc[4 * v4] = (acc[4 * v4] + y.x) * f;
                acc[4 * v4 + 1] = (acc[4 * v4 + 1] + y.y) * f;
                acc[4 * v4 + 2] = (acc[4 * v4 + 2] + y.z) * f;
                acc[4 * v4 + 3] = (acc[4 * v4 + 3] + y.w) * f;
            }
        }

        // O^T += V^T A^T over the keys up to this token half.
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            if (s4 < 2 * t + 2) {
                const bf16x8 ba = lds_ld<bf16x8>(lds, L_A + tr_off(i, 2 * s4 + lh));
                acc = mfma(vop[s4], ba, acc);
            }
        }
        // The partner's half of the V operand, read before this wave's
        // output rows overwrite those slots.
        if (upd) {
#pragma unroll
            for (int k = 0; k < 2; ++k) vs[2 * (1 - t) + k] = lds_ld<bf16x8>(lds, L_O + o_off(32 * t + ln, 4 * cc + 2 * k + lh));
        }
        // Output rows into the staging tile (stored at the next iteration).
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 pk = {pack_f32(acc[4 * g4], acc[4 * g4 + 1]), pack_f32(acc[4 * g4 + 2], acc[4 * g4 + 3])};
            lds_st(lds, L_O + o_off(i, 4 * cc + g4) + o_half(i, lh), pk);
        }

        // S = exp(G_last) S + K^T (exp(G_last - G) V) on this wave's key rows.
        if (upd) {
            const float a = __expf(Gl);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[bi][v] *= a;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
                for (int bi = 0; bi < 2; ++bi) {
                    const int c0 = 32 * (2 * t + bi) + 16 * (gi & 1);
                    const bf16x8 kt = cat4(lds_tr(lds, L_K + qk_tr_src(16 * s4 + 8 * lh, c0, m16)),
                                           lds_tr(lds, L_K + qk_tr_src(16 * s4 + 8 * lh + 4, c0, m16)));
                    S[bi] = mfma(kt, vs[s4], S[bi]);
                }
            }
        }
    }
    __syncthreads();  // the last chunk's output rows are staged
    if (nch > 0) store_o(nch - 1, true);

    if (last && p.sfin) {
        float *dst = p.sfin + ((int64_t)se.seq * H + h) * sl;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int dk = 32 * (2 * t + bi) + state_dim(v, lh);
                dst[dk * D + col] = S[bi][v];
            }
    }
}

__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void chunk_halves_kernel(HalvesParams hp) {
    int unit, half;
    xcd_unit_map(blockIdx.x, 2, unit, half);
    const int H = hp.c.H;
    const int s = unit / H;
    const int h = unit - s * H;
    if (s >= hp.onseg_max) return;
    const SegEntry se = oseg_at(hp, s);
    if (se.len < 0) return;
    __shared__ __attribute__((aligned(16))) char lds[L_BYTES];
    if ((threadIdx.x >> 6) & 1) halves_wave<1>(hp, se, h, half, lds);
    else halves_wave<0>(hp, se, h, half, lds);
}

}  // namespace

hipError_t launch_chunk_halves(const HalvesParams &hp, hipStream_t st) {
    if (hp.onseg_max == 0) return hipSuccess;
    // Two workgroups per (segment, head), laid out by xcd_unit_map: the grid
    // covers every unit when it is a multiple of 16.
    const int64_t units = (int64_t)hp.onseg_max * hp.c.H;
    const int64_t grid = (2 * units + 15) / 16 * 16;
    hipLaunchKernelGGL(chunk_halves_kernel, dim3((unsigned)grid), dim3(NTH), 0, st, hp);
    return hipGetLastError();
}

}  // namespace sgla
