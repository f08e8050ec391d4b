// Chunked gated delta rule with one gate per key dimension (KDA): q, k, v in
// fp32 or bf16, gates g [tokens, H, Dk] and write strengths beta [tokens, H]
// in fp32, Dk and Dv in {64, 128}, chunks of 64 tokens, fp32 state. The
// contractions run on the matrix cores in fp32 (fp32 16 x 16 x 4 MFMAs, or
// bf16 high/low pairs where noted, about 2^-16 of each term); the pairwise
// decay factors are exponentials on the vector ALUs.
//
// Per chunk (page "Formulas and code for adapting inference to GDN/KDA linear
// modules", section 1.2, the chunkwise formulas, with the gate made a vector
// over the key dims as in section 2.1's KDA branch), with G[a][d] the
// inclusive cumulative sum of g over the chunk's tokens for key dim d:
//
//   M[a][b] = sum_d K[a][d] K[b][d] exp(G[a][d] - G[b][d])        (a > b)
//   T       = (I + diag(beta) M)^-1                              (UT transform)
//   W       = T (diag(beta) K * exp(G)),   U = T diag(beta) V
//   new_v   = U - W S
//   L[a][b] = sum_d Q[a][d] K[b][d] exp(G[a][d] - G[b][d])        (a >= b)
//   O       = scale ((Q * exp(G)) S + L new_v)
//   S       = diag(exp(G_last)) S + (K * exp(G_last - G))^T new_v
//
// Three kernels, as for the scalar gate: kda_prep_kernel forms W, U,
// K * exp(G_last - G) and exp(G_last) for every (chunk, head) at once;
// kda_chain_kernel walks each (sequence, head, block of 16 value columns)
// through its chunks, leaving every chunk's start state and new_v behind; and
// kda_output_kernel forms every chunk's output at once from them. The prep and
// output kernels are persistent, one workgroup per CU over the (chunk, head)
// items, each loading the next item's rows while it works on the current one.
//
// The pairwise factors exp(G[a][d] - G[b][d]) of M and L are never formed as
// exp(G[a]) exp(-G[b]), which overflows once a chunk's gates sum past about
// -88. Between block I (queries a) and an earlier token b they are split at
// the block's first token c, exp(G[a] - G[c]) exp(G[c] - G[b]), two factors
// that each lie in (0, 1] when g <= 0, so every block pair costs one
// exponential per element and token rather than per pair; the products run
// on the matrix cores (bf16 high/low pairs for bf16 inputs, fp32 for fp32).
// Inside block I the same split gives a factor exp(G[c] - G[b]) >= 1 for its
// own keys b >= c, which is safe while the gates of the block span little
// (kSplitSpan); the diagonal blocks then run the same way, and a chunk where
// some block spans more takes their pairwise factors directly instead. When
// the whole chunk's gates stay within kSplitSpan of its middle token r, one
// split at r serves every pair: 64 decayed rows of each kind per chunk, and
// all ten blocks on or below the diagonal in one pass. T is inverted in 16 x 16 blocks: each
// diagonal block by back substitution on one wave, the blocks below it block
// row by block row, T_IJ = -T_II sum_K A_IK T_KJ, on fp32 MFMAs.
#include "mfma_tile.h"

namespace sgla {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool B>
struct Tag {
    static constexpr bool value = B;
};

// Stores through a buffer resource: past its range (an empty range included)
// they are dropped. The prep kernel gives every path through an item the same
// stores this way, so that the compiler's waits on the next item's loads count
// them exactly instead of waiting for every store in flight.
__device__ __forceinline__ void st_f4(buf_t r, uint32_t off, float4 v) {
    buf_st16(r, off, u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
}
__device__ __forceinline__ void st_f1(buf_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}

constexpr int KC = kChunk;  // tokens per chunk
constexpr int KP = KC + 1;  // padded token stride of transposed tiles
constexpr int XR = KC + 16; // rows of decayed queries and keys per block row (DecayTile)

// The diagonal 16 x 16 blocks of M and L are split at their first token c
// when every |G[t][d] - G[c][d]| over the block's tokens t stays within this
// span: each factor then lies within exp(+-40), finite and normal in fp32 and
// bf16, and each product term keeps about 2^-16 of its value as between
// blocks. A chunk where some block spans more takes the diagonal blocks'
// exponents pair by pair.
constexpr float kSplitSpan = 40.f;

// G: inclusive cumulative sums over a chunk's tokens, one wave per key dim
// (lane = token), for the tile Gt[DK][KP] of the chunk's gates. Sets *far
// when some token's G leaves the chunk's middle value G[KC / 2] by more than
// kSplitSpan (the writes race benignly: all store 1). Wave w takes key dims
// w, w + NT / 64, ...: all its columns are read first, so that their
// independent scans interleave.
template <int DK, int NT>
__device__ __forceinline__ void gate_prefix(float (*Gt)[KP], int w, int l, int *far) {
    constexpr int NW = NT / 64, ND = DK / NW;
    float x[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) x[i] = Gt[w + NW * i][l];
    bool span = false;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        x[i] = wave_prefix_sum(x[i]);
        span |= fabsf(x[i] - lane_value(x[i], KC / 2)) > kSplitSpan;
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) Gt[w + NW * i][l] = x[i];
    if (span) *far = 1;
}

// Sets *wide when some token's G leaves its 16-token block's first value by
// more than kSplitSpan (read from the tile Gt after gate_prefix; thread i of
// NT takes elements i, i + NT, ...). Only chunks that are not split at one
// reference token need it.
template <int DK, int NT>
__device__ __forceinline__ void block_spans(const float (*Gt)[KP], int tid, int *wide) {
    bool big = false;
#pragma unroll 4
    for (int i = tid; i < DK * KC; i += NT) {
        const int d = i / KC, t = i - d * KC;
        big |= fabsf(Gt[d][t] - Gt[d][t & ~15]) > kSplitSpan;
    }
    if (big) *wide = 1;
}

// Per chunk and head workspace tile, in floats: W, then K * exp(G_last - G),
// then U, each as fp32 MFMA operand images (below), then exp(G_last) [Dk].
//
// The chain's products are fp32 16 x 16 x 4 MFMAs: lane l = 16 kk + r
// supplies A[r][kk] and B[kk][r] and receives D[4 kk + v][r] in element v.
// Four of them cover 16 k values, MFMA k4 taking k = 4 kk + k4 for lane
// group kk, so each lane's operands for the four are one float4 and an
// accumulator quad is already the B operand of the next product. The images
// hold those float4s in lane order (1 KiB per 16 x 16 block):
//   W   [tok block tt][key block b][lane]  = W[16 tt + r][16 b + 4 kk .. +3]
//   Kd  [key block b][tok block tt][lane]  = Kd[16 tt + 4 kk .. +3][16 b + r]
//   U   [tok block tt][col block cb][lane] = U[16 tt + 4 kk .. +3][16 cb + r]
// and the chain leaves, per chunk, the start state and new_v likewise:
//   S   [key block b][col block cb][lane]  = S[16 b + 4 kk .. +3][16 cb + r]
//   nv  [tok block tt][col block cb][lane] = new_v[16 tt + 4 kk .. +3][16 cb + r]
__host__ __device__ constexpr int64_t tile_floats(int dk, int dv) {
    return 2 * (int64_t)KC * dk + (int64_t)KC * dv + dk;
}

__device__ __forceinline__ int64_t tile_index(const KdaParams &p, int64_t s, int h) {
    return (s * p.c.H + h);
}

// 16 bytes of a row as floats: 8 bf16 or 4 fp32 values.
template <typename Tin>
__device__ __forceinline__ void load_piece(const uint4 u, float *out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (sizeof(Tin) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = __uint_as_float(w[e] << 16);
            out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(w[e]);
    }
}

// bf16 tiles of rows of DK values for the 16 x 16 x 32 MFMA operands:
// 16-byte chunk c of row r sits at chunk c ^ (r mod chunks-per-row), so the
// 16 rows one operand read touches fall in different banks.
template <int DK>
__device__ __forceinline__ int brow_off(int r, int c) {
    constexpr int NC = DK / 8;
    return r * (DK * 2) + ((c ^ (r & (NC - 1))) << 4);
}

// 16 x 16 block of P = X_a X_b^T over DK (rows 16 ra0 .. and 16 rb0 .. of
// two bf16 hi/lo tile pairs), on one wave: hi hi + hi lo + lo hi, about 2^-16
// of each product. Lane (g, lc) gets P[16 ra0 + lc][16 rb0 + 4 g + r] in
// acc[r] (16 x 16 x 32 MFMA: both operands name row lc of their block and
// k = 32 ks + 8 g .. + 7; the result is C[4 g + r][lc], C = B-block x A-block).
template <int DK>
__device__ __forceinline__ f32x4 block_product(const char *ahi, const char *alo, int ra0, const char *bhi,
                                               const char *blo, int rb0, int l) {
    const int lc = l & 15, g = l >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const int oa = brow_off<DK>(16 * ra0 + lc, 4 * ks + g), ob = brow_off<DK>(16 * rb0 + lc, 4 * ks + g);
        const bf16x8 ah = lds_ld<bf16x8>(ahi, oa), al = lds_ld<bf16x8>(alo, oa);
        const bf16x8 bh = lds_ld<bf16x8>(bhi, ob), bl = lds_ld<bf16x8>(blo, ob);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, ah, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, al, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl, ah, acc, 0, 0, 0);
    }
    return acc;
}
// Both blocks from one tile pair.
template <int DK>
__device__ __forceinline__ f32x4 block_product(const char *hi, const char *lo, int ra0, int rb0, int l) {
    return block_product<DK>(hi, lo, ra0, hi, lo, rb0, l);
}

// Two floats as bf16 high parts (truncated) and low parts (the rounded
// remainders), each pair packed into one word, element 0 in the low half.
__device__ __forceinline__ void hilo2(const float *x, uint32_t &hi, uint32_t &lo) {
    const uint32_t u0 = __float_as_uint(x[0]), u1 = __float_as_uint(x[1]);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    lo = pack_f32(x[0] - __uint_as_float(u0 & 0xffff0000u), x[1] - __uint_as_float(u1 & 0xffff0000u));
}

// The value, opaque to the compiler: index math derived from it inside an
// item loop is formed there, instead of being hoisted out of the loop and
// spilled (the persistent kernels keep the next item's rows and operand
// images live across their loops).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// fp32 tiles of rows of DK values: 16-byte chunk c of row r sits at chunk
// c ^ (r mod 16), so the 16 rows one operand read touches fall in different
// banks.
template <int DK>
__device__ __forceinline__ int frow_off(int r, int c) {
    return r * (DK * 4) + ((c ^ (r & 15)) << 4);
}

// NR rows of decayed queries or keys for the pairwise products. For bf16
// inputs (HL) a bf16 high tile and, NR * DK * 2 bytes on, a low tile, whose
// products (block_product) keep about 2^-16 of each term; for fp32 inputs
// one fp32 tile, whose products run on fp32 16 x 16 x 4 MFMAs and round only
// in the accumulation. In the bf16 tiles 16-byte chunk c = 4 ks + kk of a
// row holds the values 32 ks + 4 kk .. +3 and 32 ks + 16 + 4 kk .. +3: the
// k order in which a lane of the start-state image holds its blocks 2 ks and
// 2 ks + 1, so that a tile of queries is also the A operand of (Q exp G) S_in
// (and every product of two tiles sums over the same k).
template <int DK, bool HL, int NR>
struct DecayTile {
    static constexpr int BYTES = HL ? 2 * NR * DK * 2 : NR * DK * 4;
    char *t;
    // Values d and d + 1 (d even) of row r.
    __device__ __forceinline__ void put2(int r, int d, const float *x) const {
        if constexpr (HL) {
            uint32_t hi, lo;
            hilo2(x, hi, lo);
            const int c = 4 * (d >> 5) + ((d >> 2) & 3), e = 4 * ((d >> 4) & 1) + (d & 3);
            const int off = brow_off<DK>(r, c) + 2 * e;
            *reinterpret_cast<uint32_t *>(t + off) = hi;
            *reinterpret_cast<uint32_t *>(t + NR * DK * 2 + off) = lo;
        } else {
            *reinterpret_cast<float2 *>(t + frow_off<DK>(r, d >> 2) + 4 * (d & 3)) = make_float2(x[0], x[1]);
        }
    }
};

// The 16 x 16 block P[16 ra0 + i][16 rb0 + j] = sum_d A[16 ra0 + i][d]
// B[16 rb0 + j][d] on one wave: lane (g, lc) gets P[16 ra0 + lc][16 rb0 +
// 4 g + r] in acc[r]. For fp32 tiles the k order of MFMA k4 of 16-value
// step j is 16 j + 4 g + k4 for lane group g (one float4 per operand and
// step); lane 16 g + lc supplies key row lc as A and query row lc as B, and
// receives D[4 g + r][lc].
template <int DK, bool HL, int NA, int NB>
__device__ __forceinline__ f32x4 tile_block(const DecayTile<DK, HL, NA> &A, int ra0, const DecayTile<DK, HL, NB> &B,
                                            int rb0, int l) {
    if constexpr (HL) {
        return block_product<DK>(A.t, A.t + NA * DK * 2, ra0, B.t, B.t + NB * DK * 2, rb0, l);
    } else {
        const int lc = l & 15, g = l >> 4;
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < DK / 16; ++j) {
            const float4 a = lds_ld<float4>(A.t, frow_off<DK>(16 * ra0 + lc, 4 * j + g));
            const float4 b = lds_ld<float4>(B.t, frow_off<DK>(16 * rb0 + lc, 4 * j + g));
            f32x4 &x = (j & 1) ? x1 : x0;
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(b.x, a.x, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(b.y, a.y, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(b.z, a.z, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(b.w, a.w, x, 0, 0, 0);
        }
        return x0 + x1;
    }
}

// A chunk's rows of a [tokens, H, W] tensor, held in registers as raw
// 16-byte pieces (PT per thread): load() issues the loads and returns at
// once, store() converts to fp32 and writes the tile to LDS as
// tile[col][row] (TR) or tile[row][col]. The persistent kernels load the next
// item's rows while they work on the current one. The loads go through a
// buffer resource whose range ends at row n, so rows past it read as zeros
// with no branch, and every path issues the same loads (which keeps the
// compiler's waits on them exact). Offsets stay below 2^31 bytes for
// H <= 65536 and W <= 128 fp32.
template <typename Tin, int W, int NT>
struct Rows {
    static constexpr int PE = 16 / sizeof(Tin);  // elements per piece
    static constexpr int PR = W / PE;            // pieces per row
    static constexpr int PT = KC * PR / NT;
    static_assert(KC * PR % NT == 0, "whole pieces per thread");
    // A wave's 64 pieces cover PE rows of 64 / PE pieces each: element e of
    // lane (row i, piece j) then lands in LDS word (PE j + e) * S + i or
    // i * S + PE j + e, S = 1 mod 64, whose bank PE j + i + e differs across
    // the wave's lanes; the global reads stay whole runs of 64 / PE pieces.
    static constexpr int PW = 64 / PE;  // pieces per wave row
    static constexpr int RG = KC / PE;  // row groups
    static_assert(PR % PW == 0 && KC % PE == 0, "whole wave blocks");
    __device__ __forceinline__ static void piece(int idx, int &a, int &pc) {
        const int wv = idx >> 6, lane = idx & 63;
        a = PE * (wv % RG) + lane / PW;
        pc = PW * (wv / RG) + lane % PW;
    }
    u32x4 r[PT];
    __device__ __forceinline__ void load(const Tin *base, int64_t tok0, int H, int h, int n, int tid) {
        const int bytes = n > 0 ? ((n - 1) * H * W + W) * (int)sizeof(Tin) : 0;
        const buf_t rs = buf_rsrc(base + (tok0 * H + h) * W, bytes);
#pragma unroll
        for (int m = 0; m < PT; ++m) {
            int a, pc;
            piece(m * NT + tid, a, pc);
            r[m] = buf_ld16(rs, (uint32_t)((a * H * W + pc * PE) * (int)sizeof(Tin)));
        }
    }
    // As store<false, STRIDE>, row a multiplied by scale[a] (one rounding).
    template <int STRIDE>
    __device__ __forceinline__ void store_scaled(float *tile, int tid, const float *scale) const {
#pragma unroll
        for (int m = 0; m < PT; ++m) {
            int a, pc;
            piece(m * NT + tid, a, pc);
            float f[PE];
            load_piece<Tin>(make_uint4(r[m][0], r[m][1], r[m][2], r[m][3]), f);
            const float sa = scale[a];
#pragma unroll
            for (int e = 0; e < PE; ++e) tile[a * STRIDE + pc * PE + e] = f[e] * sa;
        }
    }
    template <bool TR, int STRIDE>
    __device__ __forceinline__ void store(float *tile, int tid) const {
#pragma unroll
        for (int m = 0; m < PT; ++m) {
            int a, pc;
            piece(m * NT + tid, a, pc);
            float f[PE];
            load_piece<Tin>(make_uint4(r[m][0], r[m][1], r[m][2], r[m][3]), f);
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                const int col = pc * PE + e;
                if (TR) tile[col * STRIDE + a] = f[e];
                else tile[a * STRIDE + col] = f[e];
            }
        }
    }
};

// A (chunk, head) item of the persistent kernels: item = s H + h.
// len < 0 marks a table row with no segment; past the last item len is -1.
// TAB: the segments come from the device table (packed sequences); without
// it they are arithmetic (B sequences of T tokens) and decoding an item loads
// nothing, which leaves the compiler's waits in the item loop exact (a table
// load merged into the loop would make it wait for every store in flight).
struct Item {
    int s, h, n, len;
    int64_t tok0;
};
template <bool TAB>
__device__ __forceinline__ Item item_at(const KdaParams &p, int64_t item, int64_t nitems) {
    Item it{0, 0, 0, -1, 0};
    if (item < nitems) {
        it.s = (int)(item / p.c.H);
        it.h = (int)(item - (int64_t)it.s * p.c.H);
        SegEntry se;
        if constexpr (TAB) {
            se = seg_at(p.c, it.s);
        } else {
            const int n = it.s / p.c.nps, j = it.s - n * p.c.nps;
            const int rem = p.c.T - j * kChunk;
            se.tok0 = (int64_t)n * p.c.T + (int64_t)j * kChunk;
            se.len = rem < kChunk ? rem : kChunk;
        }
        it.len = se.len;
        it.n = se.len > 0 ? se.len : 0;
        it.tok0 = se.tok0;
    }
    return it;
}

// ---- prep: persistent over the (chunk, head) items, one workgroup per CU;
// the next item's k, g rows and beta load into registers while the current
// one is worked on, and its v rows once the current A is formed. A comes from
// decayed-key tiles on the matrix cores: split at the chunk's middle token
// when its gates allow, else block row by block row (with the diagonal
// blocks pair by pair when a block's gates span too far).
template <typename Tin, int DK, int DV, bool TAB>
__global__ __launch_bounds__(512) void kda_prep_kernel(KdaParams p, int64_t nitems) {
    constexpr int NT = 512;
    constexpr int MP = KC + 4;         // row stride of A/T: 16-byte aligned rows
    __shared__ float Kt[DK][KP];       // K^T; later (diag(beta) K * exp(G))^T
    __shared__ float Gt[DK][KP];       // G^T
    // diag(beta) V, staged once A is formed (before, the space of decayed keys)
    __shared__ __attribute__((aligned(16))) float Vs[KC][DV + 1];
    __shared__ __attribute__((aligned(16))) float Ms[KC][MP];  // A = diag(beta) M below the diagonal
    // K decayed to a reference token, XR rows of a DecayTile; later the
    // blocks of T (10 blocks of 16 rows x 20 floats).
    constexpr int XT = 2 * XR * DK * 2, XTB = 10 * 16 * 20 * 4;
    __shared__ __attribute__((aligned(16))) char Xb[XT > XTB ? XT : XTB];
    constexpr bool HL = sizeof(Tin) == 2;
    const DecayTile<DK, HL, XR> X{Xb};
    static_assert(X.BYTES <= (int)sizeof(Xb), "the decayed rows fit their space");
    // One reference token per chunk needs a second tile of KC rows: the space
    // of diag(beta) V, where it fits (not at Dk = 128 with Dv = 64).
    constexpr bool kOneRef = DecayTile<DK, HL, KC>::BYTES <= (int)sizeof(Vs);
    __shared__ float bs[KC];
    __shared__ int wide, far;  // gate spans past kSplitSpan (block_spans, gate_prefix)
    static_assert(sizeof(Kt) + sizeof(Gt) + sizeof(Vs) + sizeof(Ms) + sizeof(Xb) + sizeof(bs) + 2 * sizeof(int) <=
                      kLdsPerCU,
                  "the workgroup must fit one CU's LDS");
    const int H = p.c.H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;  // w: one value per wave
    const Tin *__restrict__ kg = static_cast<const Tin *>(p.c.k);
    const Tin *__restrict__ vg = static_cast<const Tin *>(p.c.v);

    // Rows past a chunk's end are zeros (zero gate, beta, key).
    Rows<Tin, DK, NT> rk;
    Rows<float, DK, NT> rg;
    Rows<Tin, DV, NT> rv;
    float rb = 0.f;
    // k, g and beta rows are staged at the item's top; v rows once A is
    // formed, so their loads follow later.
    auto fetch_kg = [&](int64_t item) {
        const Item it = item_at<TAB>(p, item, nitems);
        rk.load(kg, it.tok0, H, it.h, it.n, tid);
        rg.load(p.c.g, it.tok0, H, it.h, it.n, tid);
        rb = buf_ld_f32(buf_rsrc(p.beta + it.tok0 * H + it.h, it.n > 0 ? (it.n - 1) * H * 4 + 4 : 0),
                        (uint32_t)((tid & (KC - 1)) * H * 4));
    };
    auto fetch_v = [&](int64_t item) {
        const Item it = item_at<TAB>(p, item, nitems);
        rv.load(vg, it.tok0, H, it.h, it.n, tid);
    };
    fetch_kg(blockIdx.x);
    fetch_v(blockIdx.x);
    // The first item's loads complete before the loop, so that the waits at
    // its top count only the next item's loads and the stores issued after
    // them (and never wait for the stores).
#pragma unroll
    for (int m = 0; m < rk.PT; ++m) settle(rk.r[m]);
#pragma unroll
    for (int m = 0; m < rg.PT; ++m) settle(rg.r[m]);
#pragma unroll
    for (int m = 0; m < rv.PT; ++m) settle(rv.r[m]);
    settle(rb);
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
    const Item it = item_at<TAB>(p, item, nitems);
    // Without the table every item has a segment (len >= 0; T = 0 gives an
    // empty one whose tile the chain still reads).
    if (TAB && it.len < 0) {
        fetch_kg(item + gridDim.x);
        fetch_v(item + gridDim.x);
        continue;
    }
    const int s = it.s, h = it.h;
    if (tid == 0) wide = far = 0;  // the last item read them before its final barrier
    bs[tid & (KC - 1)] = rb;  // eight threads per token write the same value
    rk.template store<true, KP>(&Kt[0][0], tid);
    rg.template store<true, KP>(&Gt[0][0], tid);
    fetch_kg(item + gridDim.x);
    __syncthreads();
    gate_prefix<DK, NT>(Gt, w, l, &far);
    __syncthreads();
    const int tix = opaque(tid);

    // A from one reference token r = KC / 2 for the whole chunk, when every
    // |G[t][d] - G[r][d]| stays within kSplitSpan: K exp(G - G_r) (tokens as
    // a) in Xb, K exp(G_r - G) (tokens as b) in the space of diag(beta) V,
    // and the 10 blocks on or below the diagonal in one pass, wave w taking
    // blocks w and w + 8 (block I (I + 1) / 2 + J is (I, J)).
    bool one_ref = false;
    if constexpr (kOneRef) one_ref = __builtin_amdgcn_readfirstlane(far) == 0;
    if (one_ref) {
        constexpr int RP = KC * DK / 2 / NT;  // dim pairs per thread
        constexpr int R = KC / 2;
        const DecayTile<DK, HL, KC> Xa{Xb}, Xc{reinterpret_cast<char *>(&Vs[0][0])};
#pragma unroll
        for (int m = 0; m < RP; ++m) {
            const int i = m * NT + tix, a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
            float xa[2], xc[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float kv = Kt[d + e][a], ex = Gt[d + e][a] - Gt[d + e][R];
                xa[e] = kv * __expf(ex);
                xc[e] = kv * __expf(-ex);
            }
            Xa.put2(a, d, xa);
            Xc.put2(a, d, xc);
        }
        __syncthreads();
        for (int bi = w; bi < 10; bi += NT / 64) {
            const int I = bi < 1 ? 0 : bi < 3 ? 1 : bi < 6 ? 2 : 3, J = bi - I * (I + 1) / 2;
            const f32x4 acc = tile_block(Xa, I, Xc, J, l);
            // On the diagonal A keeps b = 16 J + g4 + v < a = 16 I + lc.
            const int lc = l & 15, g4 = 4 * (l >> 4), a = 16 * I + lc;
            const bool dg = I == J;
            const float ba = bs[a];
            *reinterpret_cast<float4 *>(&Ms[a][16 * J + g4]) =
                make_float4(!dg || g4 < lc ? ba * acc[0] : 0.f, !dg || g4 + 1 < lc ? ba * acc[1] : 0.f,
                            !dg || g4 + 2 < lc ? ba * acc[2] : 0.f, !dg || g4 + 3 < lc ? ba * acc[3] : 0.f);
        }
    } else {
        // A inside the diagonal 16 x 16 blocks (a > b): split at the block's
        // first token with the blocks below (when the gates allow), else here,
        // one pair per thread with its exponent taken directly.
        block_spans<DK, NT>(Gt, tix, &wide);
        __syncthreads();
        const bool split = __builtin_amdgcn_readfirstlane(wide) == 0;
        if (!split) {
            for (int i = tix; i < 4 * 120; i += NT) {
                const int blk = i / 120, r = i - blk * 120;
                int ai = 1;
                while ((ai + 1) * ai / 2 <= r) ++ai;
                const int a = 16 * blk + ai, b = 16 * blk + (r - ai * (ai - 1) / 2);
                float acc = 0.f;
                for (int d = 0; d < DK; ++d) acc = fmaf(Kt[d][a] * Kt[d][b], __expf(Gt[d][a] - Gt[d][b]), acc);
                Ms[a][b] = bs[a] * acc;
            }
        }
        // A by block row I: tokens b < c = 16 I, and with the split block I's own
        // tokens, against block I's, split at c. The decayed keys go to the rows
        // of X: rows below c hold K exp(G_c - G) (keys b = row), rows c .. c + 15
        // K exp(G - G_c) (block I as a), rows c + 16 .. c + 31 K exp(G_c - G)
        // (block I as b = row - 16); one wave per 16 x 16 block on the matrix
        // cores.
        for (int I = split ? 0 : 1; I < 4; ++I) {
            const int c = 16 * I, nr = c + (split ? 32 : 16);
            __syncthreads();  // the previous block row's products are done with the tiles
            for (int i = tix; i < nr * DK / 2; i += NT) {
                const int a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
                const bool qry = a >= c && a < c + 16;
                const int t = a < c + 16 ? a : a - 16;
                float x[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float ex = qry ? Gt[d + e][t] - Gt[d + e][c] : Gt[d + e][c] - Gt[d + e][t];
                    x[e] = Kt[d + e][t] * __expf(ex);
                }
                X.put2(a, d, x);
            }
            __syncthreads();
            const int lc = l & 15, g4 = 4 * (l >> 4), a = c + lc;
            if (w < I) {
                const f32x4 acc = tile_block(X, I, X, w, l);
                const float ba = bs[a];
                *reinterpret_cast<float4 *>(&Ms[a][16 * w + g4]) =
                    make_float4(ba * acc[0], ba * acc[1], ba * acc[2], ba * acc[3]);
            } else if (split && w == I) {
                // Keys b = c + g4 + r of the block itself; A keeps b < a.
                const f32x4 acc = tile_block(X, I, X, I + 1, l);
                const float ba = bs[a];
                *reinterpret_cast<float4 *>(&Ms[a][c + g4]) =
                    make_float4(g4 < lc ? ba * acc[0] : 0.f, g4 + 1 < lc ? ba * acc[1] : 0.f,
                                g4 + 2 < lc ? ba * acc[2] : 0.f, g4 + 3 < lc ? ba * acc[3] : 0.f);
            }
        }
    }
    __syncthreads();
    // diag(beta) V, in the space of the decayed keys now that A is formed;
    // then the next item's v rows.
    rv.template store_scaled<DV + 1>(&Vs[0][0], tid, bs);
    fetch_v(item + gridDim.x);

    float *tile = p.tiles + tile_index(p, s, h) * tile_floats(DK, DV);
    // T = (I + A)^-1 in 16 x 16 blocks, kept in the space of the decayed rows
    // (free once A is formed): the ten blocks (I, J), J <= I, rows of 80 bytes
    // (20 floats: the 16 rows of a block start 4 banks apart). W and U read
    // them there.
    constexpr int TBR = 20;                         // floats per block row
    constexpr int TBF = 16 * TBR;                   // floats per block
    float *tb = reinterpret_cast<float *>(Xb);      // 10 blocks = 12.5 KiB
    static_assert(10 * TBF * 4 <= (int)sizeof(Xb), "T blocks exceed the tile space");
    auto tbo = [](int I, int J) { return (I * (I + 1) / 2 + J) * TBF; };
    // The item's tile as a buffer (bytes), and an empty one for the stores
    // that only balance the paths.
    const buf_t rtile = buf_rsrc(tile, (int)(tile_floats(DK, DV) * 4));
    const buf_t rnone = buf_rsrc(tile, 0);
    constexpr int KDQ = KC / 4 * DK / (NT - 256);  // Kd image float4s per thread of waves 4..7
    if (w < 4) {
    if (l < 16) {
        // Diagonal block w, row l of T_ww = (I + A_ww)^-1: y with
        // (I + A_ww)^T y = e_l, by back substitution (once y_j is final it
        // takes A[j][m] y_j out of every y_m, m < j; 15 dependent steps).
        float y[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) y[m] = m == l ? 1.f : 0.f;
#pragma unroll
        for (int j = 15; j >= 1; --j) {
#pragma unroll
            for (int mq = 0; mq < j; mq += 4) {
                const float4 a = *reinterpret_cast<const float4 *>(&Ms[16 * w + j][16 * w + mq]);
                if (mq + 0 < j) y[mq + 0] = fmaf(-a.x, y[j], y[mq + 0]);
                if (mq + 1 < j) y[mq + 1] = fmaf(-a.y, y[j], y[mq + 1]);
                if (mq + 2 < j) y[mq + 2] = fmaf(-a.z, y[j], y[mq + 2]);
                if (mq + 3 < j) y[mq + 3] = fmaf(-a.w, y[j], y[mq + 3]);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(tb + tbo(w, w) + l * TBR + 4 * q) =
                make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
    }
        // Distinct offsets, so that the compiler keeps every one of them.
#pragma unroll
        for (int m = 0; m < KDQ; ++m) st_f4(rnone, 16u * m, make_float4(0.f, 0.f, 0.f, 0.f));
        st_f1(rnone, 16u * KDQ, 0.f);
    } else {
        // Meanwhile: K * exp(G_last - G) and exp(G_last) for the chain (rows
        // past the end have zero keys and gates, so G_last is the last row's
        // G), and X = diag(beta) K * exp(G) in place of K.
#pragma unroll
        for (int m = 0; m < KDQ; ++m) {
            const int q = m * (NT - 256) + tid - 256;
            // float4 q of the Kd image: tokens a0 .. a0 + 3, key dim d.
            const int d = 16 * (q >> 8) + (q & 15), a0 = 16 * ((q >> 6) & 3) + 4 * ((q >> 4) & 3);
            const float gl = Gt[d][KC - 1];
            float kd[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float kv = Kt[d][a0 + v], gv = Gt[d][a0 + v];
                kd[v] = kv * __expf(gl - gv);
                Kt[d][a0 + v] = kv * bs[a0 + v] * __expf(gv);
            }
            st_f4(rtile, (uint32_t)(KC * DK + 4 * q) * 4u, make_float4(kd[0], kd[1], kd[2], kd[3]));
        }
        // exp(G_last) of key dim tid - 256; threads past Dk store out of range.
        const int dl = tid - 256 < DK ? tid - 256 : DK - 1;
        st_f1(buf_rsrc(tile + 2 * KC * DK + KC * DV, DK * 4), (uint32_t)(tid - 256) * 4u, __expf(Gt[dl][KC - 1]));
    }
    __syncthreads();
    // Block rows below: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, wave J taking
    // column block J. Each 16 x 16 x 16 product is four fp32 16 x 16 x 4
    // MFMAs: lane l supplies L[l % 16][k] and R[k][l % 16] and receives
    // D[4 (l / 16) + v][l % 16] in element v, with k = 4 k4 + l / 16 in MFMA
    // k4 of the first product, and k = 4 (l / 16) + k4 in the second, whose
    // R is then X = sum_K A_IK T_KJ as the first left it in the lane.
    {
        const int lr = l & 15, lk = l >> 4;
#pragma unroll
        for (int I = 1; I < 4; ++I) {
            if (w < I) {
                const int J = w;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K)
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        const float a = Ms[16 * I + lr][16 * K + 4 * k4 + lk];
                        const float b = tb[tbo(K, J) + (4 * k4 + lk) * TBR + lr];
                        x = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, x, 0, 0, 0);
                    }
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const float a = tb[tbo(I, I) + lr * TBR + 4 * lk + k4];
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, x[k4], t, 0, 0, 0);
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) tb[tbo(I, J) + (4 * lk + v) * TBR + lr] = -t[v];
            }
            __syncthreads();
        }
    }
    // W = T X and U = T (diag(beta) V) on fp32 16 x 16 x 4 MFMAs, straight
    // into the chain's operand images. W comes out transposed, W^T = X^T T^T,
    // so that each accumulator quad is one W image float4 (4 key dims of a
    // token); U's quads are U image float4s as they stand. T is lower
    // triangular with zeros above the diagonal, so block (tt, .) sums over
    // token blocks kb <= tt only. A job is one column block of W or of U
    // (all four token blocks); wave w takes jobs w, w + 8, ...
    {
        const int lr = l & 15, lk = l >> 4;
        constexpr int NBK = DK / 16, NBV = DV / 16;
        // Jobs w, w + 8, ...; a wave with fewer real jobs runs job 0 again
        // with its stores dropped.
        constexpr int NJ = NBK + NBV, JPW = (NJ + NT / 64 - 1) / (NT / 64);
#pragma unroll
        for (int m = 0; m < JPW; ++m) {
            const int jr = w + m * (NT / 64);
            const bool real = jr < NJ;
            const int job = real ? jr : 0;
            // W's jobs (W^T = X^T T^T) and U's (U = T (beta V)) as separate
            // code, chosen once per job (the choice is the same for the wave).
            auto job4 = [&](auto wside) {
                constexpr bool ISW = decltype(wside)::value;
                const int cb = ISW ? job : job - NBK;
                // The operand that is not T, for token blocks kb = 0..3: X^T
                // [16 cb + r][16 kb + 4 kk + k4] or (beta V)[16 kb + 4 kk + k4][16 cb + r].
                float o[4][4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4)
                        o[kb][k4] = ISW ? Kt[16 * cb + lr][16 * kb + 4 * lk + k4] : Vs[16 * kb + 4 * lk + k4][16 * cb + lr];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb <= tt; ++kb) {
                        const float4 t4 = *reinterpret_cast<const float4 *>(tb + tbo(tt, kb) + lr * TBR + 4 * lk);
                        const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                        for (int k4 = 0; k4 < 4; ++k4)
                            x = ISW ? __builtin_amdgcn_mfma_f32_16x16x4f32(o[kb][k4], tv[k4], x, 0, 0, 0)
                                    : __builtin_amdgcn_mfma_f32_16x16x4f32(tv[k4], o[kb][k4], x, 0, 0, 0);
                    }
                    const uint32_t off = ISW ? (uint32_t)((tt * NBK + cb) * 64 + l) * 16u
                                             : (uint32_t)(2 * KC * DK) * 4u + (uint32_t)((tt * NBV + cb) * 64 + l) * 16u;
                    st_f4(real ? rtile : rnone, off, make_float4(x[0], x[1], x[2], x[3]));
                }
            };
            if (job < NBK) job4(Tag<true>{});
            else job4(Tag<false>{});
        }
    }
    __syncthreads();  // the next item's tiles overwrite these
    }
}

// ---- chain: one workgroup of four waves per (sequence, head, block of 16
// value columns), through the sequence's chunks in order, on fp32 MFMAs.
// Wave w holds key rows 16 b .. 16 b + 15 of the state block, for its RB
// row blocks b = RB w .. RB w + RB - 1, as accumulator quads. Per chunk:
//   1. it stores them as the chunk's start state (image layout);
//   2. new_v for token block w: U - W S over every key row, with S read from
//      LDS where each wave left its quads (as B operands, in lane order);
//   3. new_v goes to LDS and to the workspace;
//   4. S <- diag(exp(G_last)) S + Kd^T new_v on its own rows, new_v read back
//      from LDS in lane order.
// Each wave's next-chunk operands (W after step 2, Kd after step 4) are
// loaded into the registers that step just freed.
constexpr int VB = 16;
constexpr int CHAIN_NT = 256;

template <int DK, int DV>
__global__ __launch_bounds__(CHAIN_NT) void kda_chain_kernel(KdaParams p) {
    constexpr int NB = DK / 16;   // key blocks
    constexpr int RB = NB / 4;    // key blocks per wave
    constexpr int NVB = DV / VB;  // column blocks
    __shared__ float4 sbuf[NB][64];
    __shared__ float4 nbuf[4][64];
    const int H = p.c.H;
    // The NVB column blocks of a (sequence, head) share each chunk's W and
    // Kd images: they run on one XCD, through its L2.
    int nh, vb;
    xcd_unit_map(blockIdx.x, NVB, nh, vb);
    const int n = nh / H;
    const int h = nh - n * H;
    if (n >= p.c.N) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lk = l >> 4;
    const SeqEntry sq = seq_at(p.c, n);
    const int64_t sl = (int64_t)DK * DV;
    const int64_t tf = tile_floats(DK, DV);

    f32x4 sacc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 16 * (RB * w + i) + 4 * lk + v;
            sacc[i][v] = p.c.s0 ? p.c.s0[((int64_t)n * H + h) * sl + (int64_t)row * DV + vb * VB + lr] : 0.f;
        }

    // The operands are double-buffered: chunk c's sit in buffer c mod 2 and
    // are replaced by chunk c + 2's once used, so their loads have two
    // chunks' time to land (the first of a head's column blocks to ask for a
    // chunk's W and Kd fetches them from HBM).
    float4 wr0[NB], wr1[NB], ur0, ur1, kr0[RB][4], kr1[RB][4], er0[RB], er1[RB];
    auto tile_at = [&](int64_t s) {
        return reinterpret_cast<const float4 *>(p.tiles + tile_index(p, s, h) * tf);
    };
    auto load_w = [&](int64_t s, float4 (&wr)[NB], float4 &ur) {
        const float4 *t = tile_at(s);
#pragma unroll
        for (int b = 0; b < NB; ++b) wr[b] = t[(w * NB + b) * 64 + l];
        ur = t[KC * DK / 2 + (w * NVB + vb) * 64 + l];
    };
    auto load_k = [&](int64_t s, float4 (&kr)[RB][4], float4 (&er)[RB]) {
        const float4 *t = tile_at(s);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) kr[i][tt] = t[KC * DK / 4 + ((RB * w + i) * 4 + tt) * 64 + l];
            er[i] = t[(2 * KC * DK + KC * DV) / 4 + 4 * (RB * w + i) + lk];
        }
    };
    // Prefetches past the sequence's last chunk reload that chunk (unused):
    // the loads are unconditional, so every path issues the same ones.
    const int64_t last = sq.first + sq.nseg - 1;
    auto clampc = [&](int64_t s) { return s < last ? s : last; };
    if (sq.nseg > 0) {
        load_w(sq.first, wr0, ur0);
        load_k(sq.first, kr0, er0);
        load_w(clampc(sq.first + 1), wr1, ur1);
        load_k(clampc(sq.first + 1), kr1, er1);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) sbuf[RB * w + i][l] = make_float4(sacc[i][0], sacc[i][1], sacc[i][2], sacc[i][3]);
    __syncthreads();
    auto step = [&](int c, float4 (&wr)[NB], float4 &ur, float4 (&kr)[RB][4], float4 (&er)[RB]) {
        const int64_t s = sq.first + c;
        const int64_t ti = tile_index(p, s, h);
        f32x4 *sin4 = reinterpret_cast<f32x4 *>(p.sin + ti * sl);
#pragma unroll
        for (int i = 0; i < RB; ++i) __builtin_nontemporal_store(sacc[i], sin4 + ((RB * w + i) * NVB + vb) * 64 + l);
        // new_v = U - W S for tokens 16 w .. 16 w + 15 (two accumulators
        // for two independent MFMA chains).
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float4 sv = sbuf[b][l];
            f32x4 &x = (b & 1) ? x1 : x0;
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[b].x, sv.x, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[b].y, sv.y, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[b].z, sv.z, x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[b].w, sv.w, x, 0, 0, 0);
        }
        f32x4 nv;
        nv[0] = ur.x - (x0[0] + x1[0]);
        nv[1] = ur.y - (x0[1] + x1[1]);
        nv[2] = ur.z - (x0[2] + x1[2]);
        nv[3] = ur.w - (x0[3] + x1[3]);
        nbuf[w][l] = make_float4(nv[0], nv[1], nv[2], nv[3]);
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(p.nv + ti * KC * DV) + (w * NVB + vb) * 64 + l);
        load_w(clampc(s + 2), wr, ur);
        __syncthreads();  // new_v complete
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            sacc[i][0] *= er[i].x;
            sacc[i][1] *= er[i].y;
            sacc[i][2] *= er[i].z;
            sacc[i][3] *= er[i].w;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float4 nb = nbuf[tt][l];
                sacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i][tt].x, nb.x, sacc[i], 0, 0, 0);
                sacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i][tt].y, nb.y, sacc[i], 0, 0, 0);
                sacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i][tt].z, nb.z, sacc[i], 0, 0, 0);
                sacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i][tt].w, nb.w, sacc[i], 0, 0, 0);
            }
        }
        load_k(clampc(s + 2), kr, er);
#pragma unroll
        for (int i = 0; i < RB; ++i)
            sbuf[RB * w + i][l] = make_float4(sacc[i][0], sacc[i][1], sacc[i][2], sacc[i][3]);
        __syncthreads();  // the state complete; every wave is done with new_v
    };
    // Chunk pairs, then a last odd chunk on its own: with both steps of the
    // loop unconditional, every path back to its top has issued the same
    // memory operations, and the compiler's waits there count them exactly.
    int c = 0;
    for (; c + 1 < sq.nseg; c += 2) {
        step(c, wr0, ur0, kr0, er0);
        step(c + 1, wr1, ur1, kr1, er1);
    }
    if (c < sq.nseg) step(c, wr0, ur0, kr0, er0);
    if (p.c.sfin)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * (RB * w + i) + 4 * lk + v;
                p.c.sfin[((int64_t)n * H + h) * sl + (int64_t)row * DV + vb * VB + lr] = sacc[i][v];
            }
}

// ---- output: L from decayed query and key tiles on the matrix cores (split
// at the chunk's middle token when its gates allow, else block row by block
// row, with the diagonal blocks pair by pair when a block's gates span too
// far); then O = scale ((Q * exp(G)) S + L new_v) on the matrix cores, whose
// B operands are the chain's start-state and new_v images as loaded. Wave w
// takes column block w mod (Dv / 16) and TPW token blocks. Persistent over
// the (chunk, head) items, one workgroup per CU: the next item's q, k, g rows
// load into registers once the current ones are in LDS, and its images once
// the current output is formed.
template <typename Tin, int DK, int DV, bool TAB>
__global__ __launch_bounds__(512) void kda_output_kernel(KdaParams p, int64_t nitems) {
    constexpr int NT = 512;
    constexpr int NB = DK / 16;        // key blocks
    constexpr int NCB = DV / 16;       // column blocks
    constexpr int TPW = NCB / 2;       // token blocks per wave
    constexpr int LP = KC + 4;         // row stride of L: 16-byte aligned rows
    __shared__ __attribute__((aligned(16))) float Qt[DK][KP];  // Q^T; then decayed keys (one reference)
    __shared__ float Kt[DK][KP];
    __shared__ float Gt[DK][KP];
    __shared__ __attribute__((aligned(16))) float Ls[KC][LP];
    __shared__ __attribute__((aligned(16))) char Xb[2 * XR * DK * 2];  // decayed rows
    __shared__ __attribute__((aligned(16))) float eR[DK];  // exp(G_r) or 1 (below)
    __shared__ int wide, far;  // gate spans past kSplitSpan (block_spans, gate_prefix)
    static_assert(sizeof(Qt) + sizeof(Kt) + sizeof(Gt) + sizeof(Ls) + sizeof(Xb) + sizeof(eR) + 2 * sizeof(int) <=
                      kLdsPerCU,
                  "the workgroup must fit one CU's LDS");
    constexpr bool HILO = sizeof(Tin) == 2;
    // The A operands of (Q exp G) S_in: queries decayed to a reference token
    // r (G_r = 0 without one), tokens in rows.
    const DecayTile<DK, HILO, KC> Xq{Xb};
    static_assert(DecayTile<DK, HILO, XR>::BYTES <= (int)sizeof(Xb), "the decayed rows fit their space");
    static_assert(Xq.BYTES <= (int)sizeof(Qt), "the decayed keys fit in the space of Q^T");

    const int H = p.c.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lk = l >> 4;
    const int cb = w % NCB, tt0 = (w / NCB) * TPW;
    const Tin *__restrict__ qg = static_cast<const Tin *>(p.c.q);
    const Tin *__restrict__ kg = static_cast<const Tin *>(p.c.k);
    Tin *__restrict__ og = static_cast<Tin *>(p.c.out);

    Rows<Tin, DK, NT> rq, rk;
    Rows<float, DK, NT> rg;
    auto fetch_rows = [&](int64_t item) {
        const Item it = item_at<TAB>(p, item, nitems);
        rq.load(qg, it.tok0, H, it.h, it.n, tid);
        rk.load(kg, it.tok0, H, it.h, it.n, tid);
        rg.load(p.c.g, it.tok0, H, it.h, it.n, tid);
    };
    // The B operands: start-state blocks (b, cb) and new_v blocks (tt, cb).
    f32x4 sb[NB], nb[4];
    // Loaded for every item, also those with no tokens (their images hold
    // anything, and go unused), so that every path issues the same loads.
    auto fetch_ops = [&](int64_t item) {
        const Item it = item_at<TAB>(p, item, nitems);
        const int64_t ti = tile_index(p, it.s, it.h);
        const f32x4 *simg = reinterpret_cast<const f32x4 *>(p.sin + ti * DK * DV);
        const f32x4 *nimg = reinterpret_cast<const f32x4 *>(p.nv + ti * KC * DV);
#pragma unroll
        for (int b = 0; b < NB; ++b) sb[b] = __builtin_nontemporal_load(simg + (b * NCB + cb) * 64 + l);
#pragma unroll
        for (int t = 0; t < 4; ++t) nb[t] = __builtin_nontemporal_load(nimg + (t * NCB + cb) * 64 + l);
    };
    fetch_rows(blockIdx.x);
    fetch_ops(blockIdx.x);
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
    const Item it = item_at<TAB>(p, item, nitems);
    const int64_t next = item + gridDim.x;
    if (it.len <= 0) {
        fetch_rows(next);
        fetch_ops(next);
        continue;
    }
    const int h = it.h, n = it.n;
    if (tid == 0) wide = far = 0;  // the last item read them before its final barrier
    rq.template store<true, KP>(&Qt[0][0], tid);
    rk.template store<true, KP>(&Kt[0][0], tid);
    rg.template store<true, KP>(&Gt[0][0], tid);
    fetch_rows(next);
    __syncthreads();
    gate_prefix<DK, NT>(Gt, w, l, &far);
    __syncthreads();
    const int tix = opaque(tid);

    // L from one reference token r = KC / 2 for the whole chunk, when every
    // |G[t][d] - G[r][d]| stays within kSplitSpan: queries Q exp(G - G_r) in
    // Xq (which (Q exp G) S_in then takes as its A operand, with exp(G_r)
    // moved into the start state's rows), keys K exp(G_r - G) in the space of
    // Q^T once every wave is done with it, and the 10 blocks on or below the
    // diagonal in one pass, wave w taking blocks w and w + 8 (block
    // I (I + 1) / 2 + J is (I, J)). Each thread forms the dim pair d of rows
    // w, w + 8, ... (d = 2 (tid mod DK / 2) for DK = 128).
    const bool one_ref = __builtin_amdgcn_readfirstlane(far) == 0;
    if (one_ref) {
        constexpr int RP = KC * DK / 2 / NT;  // dim pairs of each row kind per thread
        constexpr int R = KC / 2;
        const DecayTile<DK, HILO, KC> Xk{reinterpret_cast<char *>(&Qt[0][0])};
#pragma unroll
        for (int m = 0; m < RP; ++m) {
            const int i = m * NT + tix, a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
            float x[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) x[e] = Qt[d + e][a] * __expf(Gt[d + e][a] - Gt[d + e][R]);
            Xq.put2(a, d, x);
        }
        if (tix < DK) eR[tix] = __expf(Gt[tix][R]);
        __syncthreads();  // every wave is done reading Q^T
#pragma unroll
        for (int m = 0; m < RP; ++m) {
            const int i = m * NT + tix, a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
            float x[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) x[e] = Kt[d + e][a] * __expf(Gt[d + e][R] - Gt[d + e][a]);
            Xk.put2(a, d, x);
        }
        __syncthreads();
        for (int bi = w; bi < 10; bi += NT / 64) {
            const int I = bi < 1 ? 0 : bi < 3 ? 1 : bi < 6 ? 2 : 3, J = bi - I * (I + 1) / 2;
            const f32x4 acc = tile_block(Xq, I, Xk, J, l);
            // On the diagonal L keeps b = 16 J + 4 lk + v <= a = 16 I + lr.
            const int b0 = 4 * lk;
            const bool dg = I == J;
            *reinterpret_cast<float4 *>(&Ls[16 * I + lr][16 * J + b0]) =
                make_float4(!dg || b0 <= lr ? acc[0] : 0.f, !dg || b0 + 1 <= lr ? acc[1] : 0.f,
                            !dg || b0 + 2 <= lr ? acc[2] : 0.f, !dg || b0 + 3 <= lr ? acc[3] : 0.f);
        }
    } else {
        // L inside the diagonal blocks: split at the block's first token with
        // the blocks below (when the gates allow), else here, one pair (a > b)
        // per thread with its exponent taken directly, the diagonal itself (no
        // decay) on the rest, zeros above it.
        block_spans<DK, NT>(Gt, tix, &wide);
        __syncthreads();
        const bool split = __builtin_amdgcn_readfirstlane(wide) == 0;
        if (!split) {
            if (tid < 4 * 120) {
                const int blk = tid / 120, r = tid - blk * 120;
                int ai = 1;
                while ((ai + 1) * ai / 2 <= r) ++ai;
                const int a = 16 * blk + ai, b = 16 * blk + (r - ai * (ai - 1) / 2);
                float acc = 0.f;
                for (int d = 0; d < DK; ++d) acc = fmaf(Qt[d][a] * Kt[d][b], __expf(Gt[d][a] - Gt[d][b]), acc);
                Ls[a][b] = acc;
                Ls[b][a] = 0.f;
            } else {
                for (int a = tid - 4 * 120; a < KC; a += NT - 4 * 120) {
                    float acc = 0.f;
                    for (int d = 0; d < DK; ++d) acc = fmaf(Qt[d][a], Kt[d][a], acc);
                    Ls[a][a] = acc;
                }
            }
        }
        // L by block row I: tokens b < c = 16 I, and with the split block I's own
        // tokens, against block I's queries, in the rows of X: rows below c
        // hold K exp(G_c - G) (keys b = row), rows c .. c + 15 Q exp(G - G_c)
        // (queries), rows c + 16 .. c + 31 K exp(G_c - G) (keys b = row - 16).
        const DecayTile<DK, HILO, XR> X{Xb};
        for (int I = split ? 0 : 1; I < 4; ++I) {
            const int c = 16 * I, nr = c + (split ? 32 : 16);
            __syncthreads();  // the previous block row's products are done with the tiles
            for (int i = tix; i < nr * DK / 2; i += NT) {
                const int a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
                const bool qry = a >= c && a < c + 16;
                const int t = a < c + 16 ? a : a - 16;
                const float *src = qry ? &Qt[0][0] : &Kt[0][0];
                float x[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float ex = qry ? Gt[d + e][t] - Gt[d + e][c] : Gt[d + e][c] - Gt[d + e][t];
                    x[e] = src[(d + e) * KP + t] * __expf(ex);
                }
                X.put2(a, d, x);
            }
            __syncthreads();
            if (w < I) {
                const f32x4 acc = tile_block(X, I, X, w, l);
                *reinterpret_cast<float4 *>(&Ls[c + lr][16 * w + 4 * lk]) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else if (split && w == I) {
                // Keys b = c + 4 lk + v of the block itself; L keeps b <= a = c + lr.
                const f32x4 acc = tile_block(X, I, X, I + 1, l);
                const int b0 = 4 * lk;
                *reinterpret_cast<float4 *>(&Ls[c + lr][c + b0]) =
                    make_float4(b0 <= lr ? acc[0] : 0.f, b0 + 1 <= lr ? acc[1] : 0.f, b0 + 2 <= lr ? acc[2] : 0.f,
                                b0 + 3 <= lr ? acc[3] : 0.f);
            }
        }
        // Q * exp(G) (no reference token) in the space of the decayed rows,
        // free once the last block row's products are done.
        __syncthreads();
        for (int i = tix; i < KC * DK / 2; i += NT) {
            const int a = i / (DK / 2), d = 2 * (i - a * (DK / 2));
            const float x[2] = {Qt[d][a] * __expf(Gt[d][a]), Qt[d + 1][a] * __expf(Gt[d + 1][a])};
            Xq.put2(a, d, x);
        }
        if (tix < DK) eR[tix] = 1.f;
    }
    __syncthreads();

    // O blocks (tt, cb): (Q exp(G - G_r)) (diag(exp(G_r)) S_in), then L new_v.
    // For bf16 inputs both run on 16 x 16 x 32 MFMAs as bf16 hi/lo (hi hi +
    // hi lo + lo hi, about 2^-16 of each term): the first takes the
    // start-state blocks 2 ks and 2 ks + 1 of each lane as one 8-value k
    // slice (Xq's k order), the second the new_v blocks 2 u and 2 u + 1
    // likewise, against L[16 tt + r][32 u + 4 kk .. +3] and L[16 tt + r]
    // [32 u + 16 + 4 kk .. +3] (zeros past block tt). For fp32 inputs they are
    // fp32 16 x 16 x 4 MFMAs, A = Xq[16 tt + r][16 b + 4 kk + k4] and
    // L[16 tt + r][16 t + 4 kk + k4]. All leave O[16 tt + 4 kk + v][16 cb + r]
    // in element v.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float4 e = *reinterpret_cast<const float4 *>(&eR[16 * b + 4 * lk]);
        sb[b][0] *= e.x;
        sb[b][1] *= e.y;
        sb[b][2] *= e.z;
        sb[b][3] *= e.w;
    }
    [[maybe_unused]] bf16x8 sh[HILO ? DK / 32 : 1], sl[HILO ? DK / 32 : 1];
    [[maybe_unused]] bf16x8 nh[2], nl[2];
    if constexpr (HILO) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const float f[8] = {sb[2 * ks][0], sb[2 * ks][1], sb[2 * ks][2], sb[2 * ks][3],
                                sb[2 * ks + 1][0], sb[2 * ks + 1][1], sb[2 * ks + 1][2], sb[2 * ks + 1][3]};
            split_bf16x8(f, sh[ks], sl[ks]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float f[8] = {nb[2 * u][0], nb[2 * u][1], nb[2 * u][2], nb[2 * u][3],
                                nb[2 * u + 1][0], nb[2 * u + 1][1], nb[2 * u + 1][2], nb[2 * u + 1][3]};
            split_bf16x8(f, nh[u], nl[u]);
        }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int tt = tt0 + j;
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HILO) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                f32x4 &x = (ks & 1) ? x1 : x0;
                const int off = brow_off<DK>(16 * tt + lr, 4 * ks + lk);
                const bf16x8 ah = lds_ld<bf16x8>(Xq.t, off), al = lds_ld<bf16x8>(Xq.t + KC * DK * 2, off);
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh[ks], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl[ks], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sh[ks], x, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 &x = (b & 1) ? x1 : x0;
                const float4 av = lds_ld<float4>(Xq.t, frow_off<DK>(16 * tt + lr, 4 * b + lk));
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, sb[b][0], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, sb[b][1], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, sb[b][2], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, sb[b][3], x, 0, 0, 0);
            }
        }
        if constexpr (HILO) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (2 * u > tt) break;
                const float4 l0 = *reinterpret_cast<const float4 *>(&Ls[16 * tt + lr][32 * u + 4 * lk]);
                const float4 l1 = 2 * u + 1 > tt
                                      ? make_float4(0.f, 0.f, 0.f, 0.f)
                                      : *reinterpret_cast<const float4 *>(&Ls[16 * tt + lr][32 * u + 16 + 4 * lk]);
                const float f[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                bf16x8 ah, al;
                split_bf16x8(f, ah, al);
                f32x4 &x = u ? x1 : x0;
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, nh[u], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, nl[u], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, nh[u], x, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t > tt) break;
                const float4 lv = *reinterpret_cast<const float4 *>(&Ls[16 * tt + lr][16 * t + 4 * lk]);
                f32x4 &x = (t & 1) ? x1 : x0;
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(lv.x, nb[t][0], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(lv.y, nb[t][1], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(lv.z, nb[t][2], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(lv.w, nb[t][3], x, 0, 0, 0);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int a = 16 * tt + 4 * lk + v;
            if (a < n) store_elem(og, ((it.tok0 + a) * H + h) * DV + 16 * cb + lr, p.c.scale * (x0[v] + x1[v]));
        }
    }
    fetch_ops(next);
    __syncthreads();  // the next item's tiles overwrite these
    }
}

template <typename Tin, int DK, int DV>
hipError_t launch_dims(const KdaParams &p, hipStream_t st) {
    // The prep and output kernels are persistent, one workgroup per CU (each
    // takes most of a CU's LDS).
    const int64_t nitems = (int64_t)p.c.nseg_max * p.c.H;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const unsigned wgs = (unsigned)std::min<int64_t>(nitems, cus);
    const bool tab = p.c.segs != nullptr || p.c.cu != nullptr;
    if (tab)
        hipLaunchKernelGGL((kda_prep_kernel<Tin, DK, DV, true>), dim3(wgs), dim3(512), 0, st, p, nitems);
    else
        hipLaunchKernelGGL((kda_prep_kernel<Tin, DK, DV, false>), dim3(wgs), dim3(512), 0, st, p, nitems);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // xcd_unit_map covers every (sequence, head) when the unit count is
    // rounded up to a multiple of the 8 XCDs; the extra ids return at once.
    const unsigned chains = (unsigned)(((int64_t)p.c.N * p.c.H + 7) / 8 * 8 * (DV / VB));
    hipLaunchKernelGGL((kda_chain_kernel<DK, DV>), dim3(chains), dim3(CHAIN_NT), 0, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (tab)
        hipLaunchKernelGGL((kda_output_kernel<Tin, DK, DV, true>), dim3(wgs), dim3(512), 0, st, p, nitems);
    else
        hipLaunchKernelGGL((kda_output_kernel<Tin, DK, DV, false>), dim3(wgs), dim3(512), 0, st, p, nitems);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_typed(const KdaParams &p, hipStream_t st) {
    if (p.dk == 128 && p.dv == 128) return launch_dims<Tin, 128, 128>(p, st);
    if (p.dk == 128 && p.dv == 64) return launch_dims<Tin, 128, 64>(p, st);
    if (p.dk == 64 && p.dv == 128) return launch_dims<Tin, 64, 128>(p, st);
    return launch_dims<Tin, 64, 64>(p, st);
}

}  // namespace

size_t kda_chunk_bytes(int dk, int dv) {
    return (size_t)(tile_floats(dk, dv) + (int64_t)KC * dv + (int64_t)dk * dv) * sizeof(float);
}

hipError_t launch_kda_chunk(const KdaParams &p, bool bf16, hipStream_t st) {
    if (p.c.nseg_max == 0 || p.c.N == 0) return hipSuccess;
    return bf16 ? launch_typed<uint16_t>(p, st) : launch_typed<float>(p, st);
}

}  // namespace sgla
