/*
 * sgla.h — C ABI of libsgla: Simple Gated Linear Attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (page "MiniCPM-SALA — Complete Blueprint", section
 * "B2 lightning-attn (Simple GLA)"): every head of every sequence keeps a
 * Dk x Dv state S. For each token t, in order,
 *
 *     S   <- exp(g_t) * S              (decay by a scalar log-decay g_t < 0)
 *     S   <- S + k_t^T v_t             (rank-1 update, S[i][j] += k_t[i] v_t[j])
 *     o_t  = scale * q_t S             (query after the update, sees token t)
 *
 * The chunked prefill computes the same thing 64 tokens at a time (page
 * "Formulas and code for adapting inference to GDN/KDA linear modules",
 * section 1.2 "Chunkwise Formulas": cumulative gate sums inside a chunk, a
 * decay-masked intra-chunk score matrix, an inter-chunk term through the
 * carried state and a state refresh, without the delta-rule terms). The decode
 * step is one token of the recurrence applied in place to a stored state (same
 * blueprint page: the state is loaded from the request's pool slot, updated,
 * and saved back).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to row-major, contiguous memory
 *     owned by the caller. The library keeps no pointer after the call.
 *   - dtype selects the element type of q, k, v and out (fp32 or bf16). g and
 *     every state are always fp32.
 *   - Supported head sizes: Dk, Dv in {64, 128}. Others give
 *     SGLA_ERR_UNSUPPORTED.
 *   - Base pointers of q, k, v, out and of every state must be 16-byte
 *     aligned; g needs 4 bytes, cu_seqlens 8, state_indices 4
 *     (SGLA_ERR_INVALID_ARG otherwise).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default
 *     stream) and the call returns without synchronising. Argument errors are
 *     reported synchronously, before anything is enqueued. Launch failures map
 *     to SGLA_ERR_HIP. Faults inside kernels surface at the caller's next
 *     synchronisation, as usual in HIP.
 *   - The library is re-entrant: it keeps no global mutable state, and it
 *     allocates no memory: scratch space comes from a caller-owned workspace
 *     (the *_ex entry points, sized by the *_workspace_size queries).
 */
#ifndef SGLA_H_
#define SGLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SGLA_OK = 0,
    SGLA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad enum      */
    SGLA_ERR_UNSUPPORTED = 2, /* a size or combination this build does not handle */
    SGLA_ERR_HIP = 3,         /* a HIP runtime call or a launch failed              */
    SGLA_ERR_WORKSPACE = 4    /* the call needs a (larger) caller workspace: see the
                                 *_workspace_size queries and the *_ex entry points */
} sgla_status;

typedef enum {
    SGLA_F32 = 0, /* q, k, v, out are float32                 */
    SGLA_BF16 = 1 /* q, k, v, out are bfloat16 (fp32 compute) */
} sgla_dtype;

/*
 * sgla_chunk_fwd — chunked prefill over whole sequences.
 *
 * Defined by the recurrence above (blueprint page, section "B2 lightning-attn
 * (Simple GLA)"), evaluated chunk by chunk (GDN/KDA page, section 1.2). The
 * interface follows the chunked call described on the GDN/KDA page, section
 * 2.1 "Operator Implementation": an initial state gathered per sequence, an
 * optional final state, and packed variable-length sequences given by
 * cumulative start offsets.
 *
 * Arguments:
 *   q, k          [B, T, H, Dk] dtype. With cu_seqlens: packed [T, H, Dk].
 *   v             [B, T, H, Dv] dtype. With cu_seqlens: packed [T, H, Dv].
 *   g             [B, T, H] fp32 log-decay per token and head (any real
 *                 value; the decay factor is exp(g)).
 *   initial_state [N, H, Dk, Dv] fp32, or NULL for zeros. N = B.
 *   out           [B, T, H, Dv] dtype, written for every token.
 *   final_state   [N, H, Dk, Dv] fp32, or NULL to skip. It may equal
 *                 initial_state (in-place update); it must not overlap any
 *                 other argument.
 *   cu_seqlens    NULL: B sequences of T tokens each.
 *                 Otherwise a device array of B + 1 int64 offsets with
 *                 cu[0] = 0, cu[i] <= cu[i+1], cu[B] = T: sequence i is the
 *                 packed tokens [cu[i], cu[i+1]). Chunks restart at every
 *                 sequence start and tokens never mix across sequences. A
 *                 zero-length sequence writes no output and its final state
 *                 equals its initial state. The offsets are read on the
 *                 device only; offsets that break the rule above are the
 *                 caller's error (results are then undefined, but every
 *                 access stays inside the buffers sized from B, T, H, Dk, Dv).
 *   B             number of sequences (>= 0; 0 is a no-op).
 *   T             tokens per sequence, or the packed total (>= 0).
 *   H             heads (1 .. 65536).
 *   Dk, Dv        head sizes of q/k and v.
 *   scale         output scale (normally 1/sqrt(Dk)).
 *   dtype         element type of q, k, v, out.
 *   stream        hipStream_t, or NULL.
 *
 * Memory: allocates nothing and takes no workspace. Every sequence is one
 * segment: one workgroup per (sequence, head), or per (sequence, head, half
 * of the value columns) for bf16 with Dk = Dv = 128. That is the fastest plan
 * when B * H fills the chip; with few long sequences, sgla_chunk_fwd_ex with a
 * workspace splits each sequence across many workgroups.
 * out must not alias q, k, v or g.
 *
 * Returns SGLA_OK, or SGLA_ERR_INVALID_ARG (null required pointer, negative
 * size, misaligned pointer, B*T*H*max(Dk,Dv) beyond 2^62, bad dtype),
 * SGLA_ERR_UNSUPPORTED (Dk or Dv not in {64, 128}, or H > 65536), SGLA_ERR_HIP.
 */
sgla_status sgla_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                           const float *initial_state, void *out, float *final_state,
                           const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                           float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_chunk_fwd_workspace_size — bytes of device workspace sgla_chunk_fwd_ex
 * uses for these sizes (0 when the call needs none).
 *
 *   varlen    0: B sequences of T tokens; 1: packed sequences (cu_seqlens),
 *             T the packed total. The size is a bound over every cu_seqlens
 *             with that B and T.
 *   prologue  0 or 1: whether q_weight will be given (the q/k prologue).
 * Other arguments as sgla_chunk_fwd. Writes *bytes (0 on error) and returns
 * SGLA_OK, SGLA_ERR_INVALID_ARG or SGLA_ERR_UNSUPPORTED under the rules of
 * sgla_chunk_fwd.
 */
sgla_status sgla_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, sgla_dtype dtype,
                                          int varlen, int prologue, size_t *bytes);

/*
 * sgla_chunk_fwd_ex — sgla_chunk_fwd with every option: the q/k prologue
 * (q_weight != NULL; see sgla_chunk_fwd_qk_norm_rope below for its arguments
 * and conditions) and a caller-owned workspace that lets long sequences be
 * split across workgroups.
 *
 * With a workspace each sequence is cut into segments. A first pass computes
 * every segment's state contribution from a zero state; these are combined in
 * order into the state each segment starts from (the recurrence regrouped:
 * the decayed initial state plus the decayed sum of outer products, blueprint
 * page, section "Why Linear Attention Loses Information"), by a scan pass or
 * by the output workgroups as they start, and the output pass runs all
 * segments at once. With packed sequences, device-side tables
 * lay the segments out from cu_seqlens.
 *
 *   workspace        device memory, 256-byte aligned, owned by the caller,
 *                    or NULL (then the call plans as sgla_chunk_fwd and needs
 *                    none). Its contents need no initialisation and are
 *                    meaningless after the call, except word 0 (int32) when
 *                    the environment sets SGLA_VALIDATE: the cu_seqlens check
 *                    of sgla_validate_cu_seqlens. Calls that overlap in time
 *                    must use different workspaces.
 *   workspace_bytes  its size; at least what sgla_chunk_fwd_workspace_size
 *                    reports for these sizes, or the call returns
 *                    SGLA_ERR_WORKSPACE without enqueuing anything.
 * All other arguments and the return codes are those of sgla_chunk_fwd.
 */
sgla_status sgla_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *initial_state, void *out, float *final_state,
                              const int64_t *cu_seqlens, const float *q_weight,
                              const float *k_weight, const int32_t *pos_offset, float theta,
                              float eps, int B, int T, int H, int Dk, int Dv, float scale,
                              sgla_dtype dtype, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * sgla_chunk_fwd_noalloc — for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): sgla_chunk_fwd_ex's split plan, with a scratch array the
 * library holds on each GPU in place of the caller's workspace. Arguments and
 * results as sgla_chunk_fwd (no prologue). It calls no allocator.
 *
 * The scratch holds at most 64 MiB per GPU (enough for the split plan of
 * B = 1, H = 32, Dk = Dv = 128 up to T = 65536); a call whose plan
 * (sgla_chunk_fwd_workspace_size) needs more returns SGLA_ERR_WORKSPACE
 * without enqueuing anything. The array is part of the library's device code
 * and is held on every GPU the library runs on until the process ends; the
 * first call on a GPU looks up its address there, with that GPU current.
 * Every call on one GPU uses the same array: calls that overlap in time on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller. Nothing in it needs clearing between calls.
 */
sgla_status sgla_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g,
                                   const float *initial_state, void *out, float *final_state,
                                   const int64_t *cu_seqlens, int B, int T, int H, int Dk, int Dv,
                                   float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_validate_cu_seqlens — checks packed-sequence offsets on the device
 * (the rules under sgla_chunk_fwd: cu[0] = 0, non-decreasing, cu[B] = T) and
 * writes to *status (device int32, 4-byte aligned) the sum of the rules
 * broken: 1 cu[0] != 0, 2 some cu[i] > cu[i+1], 4 cu[B] != T; 0 if none.
 * cu_seqlens holds B + 1 int64 values, 8-byte aligned, never NULL. Enqueued
 * on `stream`; read *status after synchronising. Returns SGLA_OK,
 * SGLA_ERR_INVALID_ARG or SGLA_ERR_HIP. Allocates nothing.
 */
sgla_status sgla_validate_cu_seqlens(const int64_t *cu_seqlens, int B, int T, int32_t *status,
                                     void *stream);

/*
 * sgla_recurrent_step — one decode token per row, state updated in place.
 *
 * Defined by one iteration of the recurrence above (blueprint page, section
 * "B2 lightning-attn (Simple GLA)": decay, outer-product update, query), with
 * the state read from and written back to the row's pool slot (same page,
 * section "Memory Architecture": the request-to-state-slot mapping of the
 * state pool).
 *
 * Arguments:
 *   q, k          [N, H, Dk] dtype.
 *   v             [N, H, Dv] dtype.
 *   g             [N, H] fp32 log-decay.
 *   state         [slots, H, Dk, Dv] fp32 pool, read and written in place.
 *   state_indices [N] int32 row -> slot map, or NULL for slot = row. Slots
 *                 must be distinct and inside [0, slots); the caller
 *                 guarantees it (the library cannot see `slots`).
 *   out           [N, H, Dv] dtype.
 *   N, H, Dk, Dv  sizes (N >= 0; 0 is a no-op).
 *   scale         output scale.
 *   dtype, stream as above.
 *
 * Returns as sgla_chunk_fwd. Allocates nothing.
 */
sgla_status sgla_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                float *state, const int32_t *state_indices, void *out, int N,
                                int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                void *stream);

/*
 * The q/k prologue variants: the same operations with q and k given BEFORE
 * the lightning layer's per-head normalisation and rotary embedding, which
 * the kernels apply as they load each tile (page "MiniCPM-SALA — Complete
 * Blueprint", section "B2 lightning-attn (Simple GLA)", the steps "QK RMSNorm
 * (per-head)" and "RoPE"). For each token and head, x being its q (or k)
 * vector of Dk = 128 values:
 *
 *     y = bf16( x / sqrt(mean(x^2) + eps) * w )      w = q_weight (k_weight),
 *                                                     one [128] vector for all heads
 *     for i < 64, with a = pos * theta^(-2i/128) radians:
 *       x'[i]      = bf16( y[i] cos a - y[i+64] sin a )
 *       x'[i + 64] = bf16( y[i+64] cos a + y[i] sin a )
 *
 * and x' takes the place of q (k) in the recurrence. The arithmetic between
 * the two bf16 roundings is fp32; the angle is reduced in fp64, so positions
 * up to 2^31 keep their accuracy. The pairing of dimension i with i + 64
 * ("rotate half"), the exact angle and eps as an argument are readings where
 * the page is silent.
 *
 * Only dtype SGLA_BF16 with Dk = 128 (and, for the chunked forward, Dv = 128)
 * is supported; other combinations return SGLA_ERR_UNSUPPORTED. theta must be
 * finite and > 0, eps finite and >= 0 (SGLA_ERR_INVALID_ARG otherwise).
 * q_weight and k_weight are device fp32 [128], 4-byte aligned, never NULL.
 */

/*
 * sgla_chunk_fwd_qk_norm_rope — sgla_chunk_fwd with the prologue.
 *
 *   pos_offset  [N] int32 device, or NULL for zeros: the position of each
 *               sequence's first token; token j of sequence n (j counted from
 *               the sequence start) has position pos_offset[n] + j. A
 *               sequence continued from an earlier call passes the number of
 *               tokens already processed.
 *   theta, eps  RoPE base (10000 on the page) and RMSNorm epsilon.
 * All other arguments and the return codes are those of sgla_chunk_fwd; it
 * allocates nothing and takes no workspace (sgla_chunk_fwd_ex with q_weight
 * takes one).
 */
sgla_status sgla_chunk_fwd_qk_norm_rope(const void *q, const void *k, const void *v,
                                        const float *g, const float *initial_state, void *out,
                                        float *final_state, const int64_t *cu_seqlens,
                                        const float *q_weight, const float *k_weight,
                                        const int32_t *pos_offset, float theta, float eps, int B,
                                        int T, int H, int Dk, int Dv, float scale,
                                        sgla_dtype dtype, void *stream);

/*
 * sgla_qk_norm_rope — the prologue alone, applied to one of q or k: the same
 * device code the chunked entry points run as they load each 64-token chunk,
 * so its output is, bit for bit, what they feed the recurrence.
 *
 *   x           [B, T, H, 128] bf16 (q or k before the prologue).
 *   weight      [128] fp32 RMSNorm weight (q_weight or k_weight).
 *   pos_offset  [B] int32 device, or NULL for zeros: token t of sequence b is
 *               at position pos_offset[b] + t.
 *   out         [B, T, H, 128] bf16; it may equal x (in place), it must not
 *               overlap it otherwise.
 *   theta, eps  as above.
 * dtype must be SGLA_BF16 and Dk 128 (SGLA_ERR_UNSUPPORTED otherwise); x and
 * out 16-byte aligned. Returns as sgla_chunk_fwd; allocates nothing.
 */
sgla_status sgla_qk_norm_rope(const void *x, const float *weight, const int32_t *pos_offset,
                              void *out, int B, int T, int H, int Dk, float theta, float eps,
                              sgla_dtype dtype, void *stream);

/*
 * sgla_recurrent_step_qk_norm_rope — sgla_recurrent_step with the prologue.
 *
 *   positions   [N] int32 device, never NULL: the position of each row's
 *               token.
 *   theta, eps  as above.
 * All other arguments and the return codes are those of sgla_recurrent_step.
 * Allocates nothing.
 */
sgla_status sgla_recurrent_step_qk_norm_rope(const void *q, const void *k, const void *v,
                                             const float *g, float *state,
                                             const int32_t *state_indices, void *out,
                                             const float *q_weight, const float *k_weight,
                                             const int32_t *positions, float theta, float eps,
                                             int N, int H, int Dk, int Dv, float scale,
                                             sgla_dtype dtype, void *stream);

/*
 * sgla_recurrent_step_ex — the decode step with every option: the state pool
 * stored in fp32 or bf16, and the q/k prologue on or off.
 *
 *   state        [slots, H, Dk, Dv] in state_dtype, read and written in place.
 *   state_dtype  SGLA_F32 or SGLA_BF16 (the pool's dtype on the blueprint
 *                page, section "B2 lightning-attn (Simple GLA)"). A bf16
 *                state is loaded, decayed, updated and read by the query in
 *                fp32 (the query sees the updated state before rounding),
 *                then stored rounded to nearest even; that halves the bytes a
 *                step moves.
 *   q_weight     NULL: no prologue (k_weight, positions, theta, eps are
 *                ignored). Otherwise the prologue of
 *                sgla_recurrent_step_qk_norm_rope, with the same conditions.
 * All other arguments and the return codes are those of sgla_recurrent_step;
 * the bf16 pool must be 16-byte aligned. Allocates nothing.
 */
sgla_status sgla_recurrent_step_ex(const void *q, const void *k, const void *v, const float *g,
                                   void *state, sgla_dtype state_dtype,
                                   const int32_t *state_indices, void *out,
                                   const float *q_weight, const float *k_weight,
                                   const int32_t *positions, float theta, float eps, int N, int H,
                                   int Dk, int Dv, float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_out_norm_gate — the output epilogue of a lightning layer.
 *
 * Defined by page "MiniCPM-SALA — Complete Blueprint", section
 * "B2 lightning-attn (Simple GLA)", step "Output Norm + Gate + Projection"
 * (without the projection). For every row r (one token, all heads
 * concatenated: width = H * Dv, 4096 on the page):
 *
 *     y   = o[r] / sqrt(mean(o[r]^2) + eps) * weight
 *     out = y * sigmoid(z[r])
 *
 * z holds the gate logits (the gate projection of the layer input, before
 * the sigmoid). With dtype SGLA_BF16, y, the gate and the product are each
 * stored in bf16 (the module outputs' dtype), the arithmetic between them is
 * fp32; with SGLA_F32 nothing is rounded beyond fp32.
 *
 * Arguments:
 *   o       [rows, width] dtype; the attention output ([B, T, H, Dv] is
 *           [B*T, H*Dv]).
 *   z       [rows, width] dtype, gate logits.
 *   weight  [width] fp32 RMSNorm weight.
 *   out     [rows, width] dtype. It may equal o (in place); it must not
 *           overlap z or weight otherwise.
 *   rows    >= 0 (0 is a no-op), < 2^31.
 *   width   a multiple of 8, at most 16384 (SGLA_ERR_UNSUPPORTED otherwise).
 *   eps     finite, >= 0.
 * o, z, weight and out must be 16-byte aligned. Returns SGLA_OK,
 * SGLA_ERR_INVALID_ARG, SGLA_ERR_UNSUPPORTED or SGLA_ERR_HIP; allocates
 * nothing.
 */
sgla_status sgla_out_norm_gate(const void *o, const void *z, const float *weight, void *out,
                               int64_t rows, int width, float eps, sgla_dtype dtype,
                               void *stream);

/*
 * The gated delta rule (GDN), the delta-rule family of linear attention that
 * page "Formulas and code for adapting inference to GDN/KDA linear modules"
 * adapts to chunked inference. Per sequence and head, with a Dk x Dv state S
 * (zeros, or the initial state) and for every token t in order (section 1.1,
 * the recursive formulas), alpha_t = exp(g[t]) and beta_t = beta[t]:
 *
 *     S   <- alpha_t S
 *     u   =  k_t^T S                       what the state returns for k_t
 *     S   <- S + beta_t k_t (v_t - u)^T    delta-rule write
 *     o_t =  scale q_t^T S
 *
 * The decay comes before the memory read, as in the page's chunkwise form
 * (section 1.2: W = T (K_beta * exp(G)) measures the correction against the
 * decayed state); the page's token-by-token pseudocode reads before the decay,
 * which the chunkwise form does not reproduce. beta is given per token and
 * head in fp32 (the page computes it as a sigmoid; any real value is
 * accepted). q and k are used as given: the page normalises keys before the
 * layer, and the caller does the same.
 */

/*
 * sgla_gdn_chunk_fwd — chunked GDN prefill over whole sequences (page
 * "Formulas and code for adapting inference to GDN/KDA linear modules",
 * section 1.2: UT transform T = (I + strictly_lower(diag(beta) K K^T *
 * Gamma))^-1, W = T (K_beta * exp(G)), U = T V_beta, new_v = U - W S per
 * chunk of 64 tokens; section 2.1 for the call: initial state per sequence,
 * final state, packed sequences by cumulative offsets).
 *
 * Arguments: as sgla_chunk_fwd, plus
 *   beta   [B, T, H] fp32 (packed [T, H] with cu_seqlens), 4-byte aligned.
 * Only dtype SGLA_BF16 with Dk = Dv = 128 and B * H <= 2^28 - 8 (B the
 * number of sequences) is supported (SGLA_ERR_UNSUPPORTED otherwise).
 *
 * Memory: the chunkwise form keeps, per chunk and head, W and new_v in bf16
 * and U in fp32 (64 KiB) in device memory between its kernels, so the call
 * needs a caller workspace: sgla_gdn_chunk_fwd returns SGLA_ERR_WORKSPACE
 * whenever there are tokens to process (use sgla_gdn_chunk_fwd_ex), and
 * otherwise (B = 0, or T = 0 with the final state copied) succeeds without
 * one. Returns as sgla_chunk_fwd.
 */
sgla_status sgla_gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, void *out,
                               float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                               int Dk, int Dv, float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_gdn_chunk_fwd_workspace_size — bytes of workspace sgla_gdn_chunk_fwd_ex
 * needs: 256 + (tables with varlen) + (chunks * H) * 64 KiB, where chunks is
 * B * ceil(T / 64), or T / 64 + B + 1 with varlen (a bound over every
 * cu_seqlens). Arguments and return codes as sgla_chunk_fwd_workspace_size.
 */
sgla_status sgla_gdn_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv,
                                              sgla_dtype dtype, int varlen, size_t *bytes);

/*
 * sgla_gdn_chunk_fwd_ex — sgla_gdn_chunk_fwd with a caller-owned workspace
 * (256-byte aligned, workspace_bytes at least the size query's answer, or
 * SGLA_ERR_WORKSPACE; contents need no initialisation; overlapping calls need
 * different workspaces; word 0 receives the cu_seqlens check under
 * SGLA_VALIDATE as for sgla_chunk_fwd_ex). Allocates nothing.
 */
sgla_status sgla_gdn_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state, void *out,
                                  float *final_state, const int64_t *cu_seqlens, int B, int T,
                                  int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * sgla_gdn_recurrent_step — one GDN decode token per row, state updated in
 * place through the row -> slot map (one iteration of the recurrence above).
 *
 * Arguments: as sgla_recurrent_step, plus
 *   beta   [N, H] fp32, 4-byte aligned.
 * dtype SGLA_F32 or SGLA_BF16; Dk, Dv in {64, 128}. The state pool is fp32.
 * Returns as sgla_recurrent_step. Allocates nothing.
 */
sgla_status sgla_gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, float *state,
                                    const int32_t *state_indices, void *out, int N, int H, int Dk,
                                    int Dv, float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_kda_chunk_fwd — chunked prefill of the gated delta rule with one gate
 * per key dimension (KDA) over whole sequences (page "Formulas and code for
 * adapting inference to GDN/KDA linear modules", section 1.2's chunkwise
 * formulas with the gate made a vector over the key dims, as section 2.1's
 * KDA branch does; section 2.1 for the call: chunk_kda takes q, k, v, g,
 * beta, an initial state per sequence, returns the final state, and packs
 * sequences by cumulative offsets). Per chunk of 64 tokens, with G[a][d] the
 * cumulative gate sum of key dim d:
 *
 *     M[a][b] = sum_d k_a[d] k_b[d] exp(G[a][d] - G[b][d])  (a > b)
 *     T = (I + diag(beta) M)^-1,  W = T (diag(beta) K * exp(G)),  U = T diag(beta) V
 *     new_v = U - W S,  O = scale ((Q * exp(G)) S + L new_v)  (L as M with q_a, a >= b)
 *     S = diag(exp(G_last)) S + (K * exp(G_last - G))^T new_v
 *
 * which equals the token-by-token recurrence of sgla_kda_recurrent_step.
 *
 * Arguments: as sgla_gdn_chunk_fwd, except
 *   g      [B, T, H, Dk] fp32 (packed [T, H, Dk] with cu_seqlens), 16-byte
 *          aligned: each token's gate per key dim. Any real values whose
 *          partial sums inside a 64-token chunk keep exp() within fp32 range.
 * dtype SGLA_F32 or SGLA_BF16 (q, k, v, out); Dk, Dv in {64, 128}; all
 * arithmetic is fp32.
 *
 * Memory: the chunkwise form keeps per chunk and head its W, U,
 * K * exp(G_last - G), new_v and start state in device memory between its
 * kernels (fp32; 192.5 KiB at Dk = Dv = 128), so the call needs a caller
 * workspace: sgla_kda_chunk_fwd returns SGLA_ERR_WORKSPACE whenever there are
 * tokens to process (use sgla_kda_chunk_fwd_ex), and otherwise (B = 0, or
 * T = 0 with the final state copied) succeeds without one. Returns as
 * sgla_chunk_fwd.
 */
sgla_status sgla_kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, void *out,
                               float *final_state, const int64_t *cu_seqlens, int B, int T, int H,
                               int Dk, int Dv, float scale, sgla_dtype dtype, void *stream);

/*
 * sgla_kda_chunk_fwd_workspace_size — bytes of workspace sgla_kda_chunk_fwd_ex
 * needs: 256 + (tables with varlen) + (chunks * H) * (2 * 64 * Dk + 64 * Dv +
 * Dk + 64 * Dv + Dk * Dv) * 4 bytes, each part rounded up to 256, where
 * chunks is B * ceil(T / 64), or T / 64 + B + 1 with varlen (a bound over
 * every cu_seqlens). Arguments and return codes as
 * sgla_chunk_fwd_workspace_size.
 */
sgla_status sgla_kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv,
                                              sgla_dtype dtype, int varlen, size_t *bytes);

/*
 * sgla_kda_chunk_fwd_ex — sgla_kda_chunk_fwd with a caller-owned workspace
 * (256-byte aligned, workspace_bytes at least the size query's answer, or
 * SGLA_ERR_WORKSPACE; contents need no initialisation; overlapping calls need
 * different workspaces; word 0 receives the cu_seqlens check under
 * SGLA_VALIDATE as for sgla_chunk_fwd_ex). Allocates nothing.
 */
sgla_status sgla_kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state, void *out,
                                  float *final_state, const int64_t *cu_seqlens, int B, int T,
                                  int H, int Dk, int Dv, float scale, sgla_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * sgla_kda_recurrent_step — one decode token per row of the gated delta rule
 * with one gate per key dimension (KDA; page "Formulas and code for adapting
 * inference to GDN/KDA linear modules", section 2.1: the recurrent kernel's
 * KDA branch loads a gate vector over the key dims and scales each state row
 * by the exponential of its own dim's gate; the rest of the step is the GDN
 * step above):
 *
 *     S[i][:] <- exp(g_t[i]) S[i][:]   (i = 0 .. Dk-1)
 *     u = k_t^T S ;  S <- S + beta_t k_t (v_t - u)^T ;  o_t = scale q_t^T S
 *
 * Arguments: as sgla_gdn_recurrent_step, except
 *   g      [N, H, Dk] fp32 (row-major, 4-byte aligned): the token's gate per
 *          key dim (any real value; the exponential must stay in fp32 range).
 * Returns as sgla_recurrent_step. Allocates nothing.
 */
sgla_status sgla_kda_recurrent_step(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, float *state,
                                    const int32_t *state_indices, void *out, int N, int H, int Dk,
                                    int Dv, float scale, sgla_dtype dtype, void *stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *sgla_status_string(sgla_status s);

/* Library version as major*10000 + minor*100 + patch. */
int sgla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGLA_H_ */
