// Chunked Simple GLA on the vector ALUs (fp32 arithmetic throughout).
//
// This is the path for fp32 inputs, and the general fallback shape for any
// supported head size. One workgroup owns one segment of one head and a block
// of 32 value columns, and walks the segment chunk by chunk (64 tokens). For a
// chunk with inclusive cumulative gate sums G_i (page "Formulas and code for
// adapting inference to GDN/KDA linear modules", section 1.2: cumulative sum of
// g, decay matrix exp(G_i - G_j) on and below the diagonal):
//
//   o_i   = scale * ( exp(G_i) * q_i S  +  sum_{j<=i} exp(G_i - G_j) (q_i . k_j) v_j )
//   S    <- exp(G_last) * S  +  sum_j exp(G_last - G_j) k_j^T v_j
//
// The diagonal j = i is included because the query reads the state after the
// token's own update (blueprint page, section "B2 lightning-attn (Simple GLA)").
// With STATE_ONLY the kernel computes only the second line from a zero state
// and stores the segment's state contribution and total log-decay.
#include "sgla_internal.h"

namespace sgla {

namespace {

constexpr int kBV = 32;  // value columns per workgroup

template <typename Tin, int DK, int DV, bool STATE_ONLY>
__global__ __launch_bounds__(256) void chunk_valu_kernel(ChunkParams p) {
    constexpr int NVB = DV / kBV;
    int unit, vb;
    xcd_unit_map(blockIdx.x, NVB, unit, vb);
    const int s = unit / p.H;
    const int h = unit - s * p.H;
    if (s >= p.nseg_max) return;
    const SegEntry se = seg_at(p, s);
    if (se.len < 0) return;
    const bool last = se.p == se.nseg - 1;
    if (STATE_ONLY && last) return;

    const Tin *__restrict__ q = static_cast<const Tin *>(p.q);
    const Tin *__restrict__ k = static_cast<const Tin *>(p.k);
    const Tin *__restrict__ v = static_cast<const Tin *>(p.v);
    Tin *__restrict__ out = static_cast<Tin *>(p.out);
    const int H = p.H;
    const int tid = threadIdx.x;
    const int col0 = vb * kBV;

    __shared__ float Qs[STATE_ONLY ? 1 : kChunk][DK + 1];
    __shared__ float Ks[kChunk][DK + 1];
    __shared__ float Vs[kChunk][kBV + 1];
    __shared__ float As[STATE_ONLY ? 1 : kChunk][kChunk + 1];
    __shared__ float Ss[DK][kBV + 1];
    __shared__ float Gs[kChunk], eGs[kChunk], eLs[kChunk];
    __shared__ float glast_s;
    static_assert(sizeof(Qs) + sizeof(Ks) + sizeof(Vs) + sizeof(As) + sizeof(Ss) + 3 * sizeof(Gs) +
                      sizeof(float) <= kLdsPerCU,
                  "the workgroup must fit one CU's LDS");

    // Carried-in state of this segment.
    const int64_t sl = (int64_t)DK * DV;
    const float *src = nullptr;
    if (!STATE_ONLY) {
        if (se.nseg == 1) src = p.s0 ? p.s0 + ((int64_t)se.seq * H + h) * sl : nullptr;
        else src = p.buf + ((int64_t)s * H + h) * sl;
    }
    for (int i = tid; i < DK * kBV; i += 256) {
        const int d = i / kBV, c = i - (i / kBV) * kBV;
        Ss[d][c] = src ? src[(int64_t)d * DV + col0 + c] : 0.f;
    }
    float gam_acc = 0.f;

    for (int c0 = 0; c0 < se.len; c0 += kChunk) {
        const int n = min(kChunk, se.len - c0);
        const int64_t t0 = se.tok0 + c0;
        for (int i = tid; i < kChunk * DK; i += 256) {
            const int r = i / DK, d = i - (i / DK) * DK;
            const int64_t off = ((t0 + r) * H + h) * DK + d;
            Ks[r][d] = r < n ? load_elem(k, off) : 0.f;
            if (!STATE_ONLY) Qs[r][d] = r < n ? load_elem(q, off) : 0.f;
        }
        for (int i = tid; i < kChunk * kBV; i += 256) {
            const int r = i / kBV, c = i - (i / kBV) * kBV;
            Vs[r][c] = r < n ? load_elem(v, ((t0 + r) * H + h) * DV + col0 + c) : 0.f;
        }
        if (tid < kChunk) {
            // Inclusive prefix sum of g over the chunk, one lane per token.
            float G = tid < n ? p.g[(t0 + tid) * H + h] : 0.f;
            for (int off = 1; off < kChunk; off <<= 1) {
                const float up = __shfl_up(G, off, kChunk);
                if (tid >= off) G += up;
            }
            const float gl = __shfl(G, kChunk - 1, kChunk);
            Gs[tid] = G;
            eGs[tid] = __expf(G);
            eLs[tid] = __expf(gl - G);
            if (tid == 0) glast_s = gl;
        }
        __syncthreads();
        const float gl = glast_s;
        gam_acc += gl;

        if (!STATE_ONLY) {
            // Decay-masked scores, scale folded in.
            {
                const int i = tid >> 2;
                for (int m = 0; m < kChunk / 4; ++m) {
                    const int j = (tid & 3) + 4 * m;
                    float a = 0.f;
                    if (j <= i && i < n) {
                        float acc = 0.f;
#pragma unroll 8
                        for (int d = 0; d < DK; ++d) acc = fmaf(Qs[i][d], Ks[j][d], acc);
                        a = p.scale * __expf(Gs[i] - Gs[j]) * acc;
                    }
                    As[i][j] = a;
                }
            }
            __syncthreads();
            // Outputs: inter-chunk term through the carried state + intra-chunk term.
            {
                const int c = tid & (kBV - 1);
                for (int m = 0; m < kChunk / 8; ++m) {
                    const int i = (tid >> 5) + 8 * m;
                    if (i >= n) continue;
                    float inter = 0.f;
#pragma unroll 8
                    for (int d = 0; d < DK; ++d) inter = fmaf(Qs[i][d], Ss[d][c], inter);
                    float o = p.scale * eGs[i] * inter;
                    for (int j = 0; j <= i; ++j) o = fmaf(As[i][j], Vs[j][c], o);
                    store_elem(out, ((t0 + i) * H + h) * DV + col0 + c, o);
                }
            }
            __syncthreads();
        }

        const bool need_update = STATE_ONLY || (c0 + kChunk < se.len) || (last && p.sfin);
        if (need_update) {
            const float a = __expf(gl);
            const int c = tid & (kBV - 1);
            for (int m = 0; m < DK / 8; ++m) {
                const int d = (tid >> 5) + 8 * m;
                float acc = 0.f;
                for (int j = 0; j < n; ++j) acc = fmaf(Ks[j][d] * eLs[j], Vs[j][c], acc);
                Ss[d][c] = fmaf(a, Ss[d][c], acc);
            }
        }
        __syncthreads();
    }

    float *dst = nullptr;
    if (STATE_ONLY) dst = p.buf + ((int64_t)s * H + h) * sl;
    else if (last && p.sfin) dst = p.sfin + ((int64_t)se.seq * H + h) * sl;
    if (dst) {
        for (int i = tid; i < DK * kBV; i += 256) {
            const int d = i / kBV, c = i - (i / kBV) * kBV;
            dst[(int64_t)d * DV + col0 + c] = Ss[d][c];
        }
    }
    if (STATE_ONLY && vb == 0 && tid == 0) p.gam[(int64_t)s * H + h] = gam_acc;
}

template <typename Tin, int DK, int DV>
hipError_t launch_t(const ChunkParams &p, bool phase_state, hipStream_t st) {
    constexpr int NVB = DV / kBV;
    const int64_t units = (int64_t)p.nseg_max * p.H;
    const int64_t units_pad = (units + 7) / 8 * 8;
    const dim3 grid((unsigned)(units_pad * NVB));
    if (phase_state)
        hipLaunchKernelGGL((chunk_valu_kernel<Tin, DK, DV, true>), grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((chunk_valu_kernel<Tin, DK, DV, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_dims(const ChunkParams &p, int Dk, int Dv, bool phase_state, hipStream_t st) {
    if (Dk == 128 && Dv == 128) return launch_t<Tin, 128, 128>(p, phase_state, st);
    if (Dk == 128 && Dv == 64) return launch_t<Tin, 128, 64>(p, phase_state, st);
    if (Dk == 64 && Dv == 128) return launch_t<Tin, 64, 128>(p, phase_state, st);
    return launch_t<Tin, 64, 64>(p, phase_state, st);
}

}  // namespace

hipError_t launch_chunk_valu(const ChunkParams &p, bool bf16, int Dk, int Dv, bool phase_state,
                             hipStream_t st) {
    if (p.nseg_max == 0) return hipSuccess;
    if (bf16) return launch_dims<uint16_t>(p, Dk, Dv, phase_state, st);
    return launch_dims<float>(p, Dk, Dv, phase_state, st);
}

}  // namespace sgla
