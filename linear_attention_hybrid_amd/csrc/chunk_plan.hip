// Segment planning and the carried-state scan of the chunked forward.
//
// A long sequence is cut into segments of whole chunks so that many
// workgroups can work on it at once. Each segment's state contribution is
// computed from a zero state (the chunk state refresh of page "Formulas and
// code for adapting inference to GDN/KDA linear modules", section 1.2, applied
// chunk after chunk), then a short sequential pass per (sequence, head)
// combines them into the state each segment starts from:
//
//     S_in(0) = S0,    S_in(j+1) = exp(Gamma_j) * S_in(j) + dS_j
//
// where Gamma_j is the sum of g over segment j and dS_j its zero-start state.
// This is the recurrence itself, regrouped: unrolling it over a segment gives
// exactly exp(Gamma_j) * S_in(j) plus the segment's own decayed outer products
// (blueprint page, section "Why Linear Attention Loses Information": the state
// is the decayed initial state plus the decayed sum of outer products).
#include "sgla_internal.h"

namespace sgla {

__global__ __launch_bounds__(256) void plan_kernel(const int64_t *__restrict__ cu, int B, int T,
                                                   int seg_len, int nseg_max,
                                                   SegEntry *__restrict__ segs,
                                                   SeqEntry *__restrict__ seqs) {
    __shared__ int32_t sbuf[256];
    __shared__ int32_t carry;
    static_assert(sizeof(sbuf) + sizeof(carry) <= kLdsPerCU, "the workgroup must fit one CU's LDS");
    const int tid = threadIdx.x;
    const int64_t ttot = cu ? (int64_t)T : (int64_t)B * T;
    if (tid == 0) carry = 0;
    __syncthreads();
    // Pass 1: segments per sequence and the exclusive prefix sum of them.
    for (int base = 0; base < B; base += 256) {
        const int n = base + tid;
        int32_t ns = 0;
        if (n < B) {
            int64_t len = cu ? cu[n + 1] - cu[n] : (int64_t)T;
            if (len < 0) len = 0;
            ns = len == 0 ? 1 : (int32_t)((len + seg_len - 1) / seg_len);
        }
        sbuf[tid] = ns;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t add = tid >= off ? sbuf[tid - off] : 0;
            __syncthreads();
            sbuf[tid] += add;
            __syncthreads();
        }
        const int32_t first = carry + sbuf[tid] - ns;
        if (n < B) {
            // Offsets that break the documented rule could ask for more rows
            // than the table has; clamp so every later access stays inside.
            int32_t room = nseg_max - first;
            if (room < 0) room = 0;
            seqs[n].first = first < nseg_max ? first : nseg_max;
            seqs[n].nseg = ns < room ? ns : room;
        }
        __syncthreads();
        if (tid == 255) carry += sbuf[255];
        __syncthreads();
    }
    const int32_t total = carry;
    // Pass 2: one table row per segment.
    for (int s = tid; s < nseg_max; s += 256) {
        SegEntry e;
        e.pad0 = 0;
        e.pad1 = 0;
        if (s >= total || B == 0) {
            e.tok0 = 0;
            e.len = -1;
            e.seq = 0;
            e.p = 0;
            e.nseg = 0;
            segs[s] = e;
            continue;
        }
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seqs[mid].first <= s) lo = mid; else hi = mid - 1;
        }
        const int n = lo;
        const int32_t p = s - seqs[n].first;
        const int64_t start = cu ? cu[n] : (int64_t)n * T;
        const int64_t len = cu ? cu[n + 1] - cu[n] : (int64_t)T;
        int64_t tok0 = start + (int64_t)p * seg_len;
        int64_t l = len - (int64_t)p * seg_len;
        if (l > seg_len) l = seg_len;
        if (l < 0) l = 0;
        if (tok0 < 0) { tok0 = 0; l = 0; }
        if (tok0 > ttot) { tok0 = ttot; l = 0; }
        if (tok0 + l > ttot) l = ttot - tok0;
        e.tok0 = tok0;
        e.len = (int32_t)l;
        e.seq = n;
        e.p = p;
        e.nseg = seqs[n].nseg;
        if (p >= e.nseg) e.len = -1;
        segs[s] = e;
    }
}

// One thread owns four consecutive state elements of one (sequence, head) and
// walks the sequence's segments in order. In place: the slot of segment j
// holds dS_j on entry, and on exit S_in(j) for every j that starts an output
// segment (j a multiple of rsub); the other slots are left as they are.
// Segments go in batches with three separate phases: all loads, then the
// combines in registers, then the stores. Keeping branches out of the first
// two phases lets a batch cost one memory latency; a store between two loads
// would make every later wait count it, and a branch between them makes the
// compiler wait for all of them.
template <int DK, int DV>
__global__ __launch_bounds__(256) void scan_kernel(ChunkParams p) {
    constexpr int kBatch = 16;
    const int nh = blockIdx.x;
    const int n = nh / p.H;
    const int h = nh - n * p.H;
    const SeqEntry se = seq_at(p, n);
    const int R = p.rsub;
    const int nout = (se.nseg + R - 1) / R;  // output segments of the sequence
    if (nout <= 1) return;
    const int nj = R * (nout - 1);  // segment states combined; S_in(nj) is the last one stored
    const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
    const int64_t stride = (int64_t)p.H * DK * DV;  // floats between segment slots
    float *slot0 = p.buf + ((int64_t)se.first * p.H + h) * DK * DV + e;
    const float *gam0 = p.gam + (int64_t)se.first * p.H + h;
    float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.s0) S = *reinterpret_cast<const float4 *>(p.s0 + ((int64_t)n * p.H + h) * DK * DV + e);
    for (int j0 = 0; j0 <= nj; j0 += kBatch) {
        // Slots past the last segment state are clamped to a valid one; the
        // states they produce are never stored.
        float4 d[kBatch];
        float lg[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int j = min(j0 + b, nj - 1);
            d[b] = *reinterpret_cast<const float4 *>(slot0 + j * stride);
            lg[b] = gam0[(int64_t)j * p.H];
        }
        float4 o[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            o[b] = S;
            const float a = __expf(lg[b]);
            S.x = fmaf(a, S.x, d[b].x);
            S.y = fmaf(a, S.y, d[b].y);
            S.z = fmaf(a, S.z, d[b].z);
            S.w = fmaf(a, S.w, d[b].w);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int j = j0 + b;
            if (j <= nj && j % R == 0) *reinterpret_cast<float4 *>(slot0 + j * stride) = o[b];
        }
    }
}

// One workgroup checks the offsets' rules and writes the bits of the broken
// ones (see launch_validate_cu).
__global__ __launch_bounds__(256) void validate_cu_kernel(const int64_t *__restrict__ cu, int B, int T,
                                                          int32_t *__restrict__ status) {
    __shared__ int32_t bits;
    if (threadIdx.x == 0) bits = 0;
    __syncthreads();
    int32_t mine = 0;
    for (int i = threadIdx.x; i < B; i += blockDim.x)
        if (cu[i] > cu[i + 1]) mine |= 2;
    if (threadIdx.x == 0) {
        if (cu[0] != 0) mine |= 1;
        if (cu[B] != (int64_t)T) mine |= 4;
    }
    if (mine) atomicOr(&bits, mine);
    __syncthreads();
    if (threadIdx.x == 0) *status = bits;
}

hipError_t launch_validate_cu(const int64_t *cu, int B, int T, int32_t *status, hipStream_t st) {
    hipLaunchKernelGGL(validate_cu_kernel, dim3(1), dim3(256), 0, st, cu, B, T, status);
    return hipGetLastError();
}

hipError_t launch_plan(const int64_t *cu, int B, int T, int seg_len, int nseg_max,
                       SegEntry *segs, SeqEntry *seqs, hipStream_t st) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, cu, B, T, seg_len, nseg_max, segs,
                       seqs);
    return hipGetLastError();
}

hipError_t launch_scan(const ChunkParams &p, int Dk, int Dv, hipStream_t st) {
    if (p.N == 0) return hipSuccess;
    const dim3 grid(p.N * p.H, (Dk * Dv) / 1024);
    if (Dk == 128 && Dv == 128) hipLaunchKernelGGL((scan_kernel<128, 128>), grid, dim3(256), 0, st, p);
    else if (Dk == 128 && Dv == 64) hipLaunchKernelGGL((scan_kernel<128, 64>), grid, dim3(256), 0, st, p);
    else if (Dk == 64 && Dv == 128) hipLaunchKernelGGL((scan_kernel<64, 128>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((scan_kernel<64, 64>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace sgla
