/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention token-mixer library.
 *
 * What the library computes is the KDA mixer described on
 *   "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches" (flozi.net),
 *   section "KDA replaces a token list with a recurrent matrix":
 * q/k/v projections of width 64 x 128, a causal width-4 short convolution with
 * SiLU per stream, normalised q and k, channel-dependent retention and a
 * delta-rule write into a per-head recurrent matrix, a read with the query, and
 * an output normalisation times a sigmoid gate before the output projection.
 * Per head, with the state S of shape dk x dv (rows are key channels):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = scale * S_t^T q_t,          alpha_t = exp(max(g_t, lower_bound)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are caller-owned DEVICE pointers (allocated by the caller, e.g. by
 *   PyTorch), except those named *_host. The library allocates no memory.
 * - Tensors are dense, row-major, last dimension fastest, unless a leading
 *   dimension ("ld", in elements) is given for the row stride.
 * - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is the
 *   null stream). Nothing synchronises the host.
 * - The return value is a kda_status. All arguments are validated on the host
 *   before anything is enqueued: on any error nothing is launched, no output
 *   is touched, and kda_last_error() returns a message. No exception crosses
 *   the ABI.
 * - Base pointers must be 16-byte aligned.
 * - Results are deterministic: no atomics, fixed reduction orders.
 * - kda_dtype selects float32 or bfloat16 storage; bfloat16 values are stored
 *   as their 16-bit patterns, rounded to nearest even by the library.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent cu_seqlens, misalignment, aliasing */
    KDA_ERR_UNSUPPORTED = -2, /* valid but not implemented here (e.g. dk != 128) */
    KDA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    KDA_ERR_HIP = -4          /* the HIP runtime reported an error on launch */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

#define KDA_VERSION 100 /* 1.0.0 */

/* ------------------------------------------------------------------------
 * kda_prefill -- the KDA core over packed variable-length sequences.
 *
 * Defined by the recurrence above (flozi.net page, section "KDA replaces a
 * token list with a recurrent matrix"; the per-layer state of 64 x 128 x 128
 * FP32 and the -5 log-retention bound are from the same section). Computed
 * chunk-wise (64 tokens for bfloat16 inputs, 32 for float32) with an exact
 * reorganisation of the recurrence; results equal the token-serial recurrence
 * up to rounding.
 *
 * q, k, g    [num_tokens, H, dk]   in_dtype. g is the natural-log retention
 *                                  (<= 0); it is clamped at lower_bound on use.
 *                                  q and k are expected unit-norm per head (the
 *                                  prologue produces them); the core does not
 *                                  normalise.
 * v          [num_tokens, H, dv]   in_dtype
 * beta       [num_tokens, H]       in_dtype, write strength in [0, 1]
 * cu_seqlens_dev / cu_seqlens_host  int32 [num_seqs + 1], the same values on
 *            device and host: cu[0] = 0, non-decreasing, cu[num_seqs] =
 *            num_tokens. Sequence n is tokens [cu[n], cu[n+1]); empty
 *            sequences are allowed (final state = initial state). Both NULL:
 *            num_seqs sequences of num_tokens / num_seqs tokens back to back
 *            (num_tokens must then be a multiple of num_seqs).
 * initial_state  float32 [num_seqs, H, dk, dv] or NULL (zero state).
 * final_state    float32 [num_seqs, H, dk, dv] or NULL (not written). May be
 *            the same pointer as initial_state (in-place update); any other
 *            overlap is rejected.
 * o          [num_tokens, H, dv]   out_dtype (float32 keeps full precision).
 * scale      read-out multiplier (1.0 for the plain S^T q read).
 * lower_bound  log-retention floor: -5 for the safe forget gate of the same
 *            section. Must lie in [-5.4, 0]: the chunk form multiplies decay
 *            factors 2^x with |x| up to 16 |lower_bound| log2(e) (one 16-token
 *            block of clamped log-retentions), which must stay within the
 *            normal float32 range. NaN or a positive floor returns
 *            KDA_ERR_INVALID_ARG, a floor below -5.4 KDA_ERR_UNSUPPORTED.
 * workspace / workspace_bytes  device scratch, caller-owned, not touching
 *            any tensor above. NULL: the single-pass form runs (one workgroup
 *            per (sequence, head) carries the state through all chunks; no
 *            scratch). With BF16 inputs and a workspace, the two-pass form runs:
 *            the chunk-local products of every chunk are computed in parallel
 *            and stored in the workspace (70.5 KiB per chunk and head, float16),
 *            then a sequential pass over the chunks carries the state. The
 *            chunks of each sequence are taken in windows of as many as the
 *            workspace holds; with more than one window a float32 state carry
 *            of num_seqs*H*64 KiB is kept at the end of the workspace. The
 *            minimum is one chunk slot per (sequence, head) plus that carry
 *            (or a slot for every chunk, if smaller); less returns
 *            KDA_ERR_WORKSPACE. kda_prefill_workspace_bytes() gives the
 *            recommended size (windows of up to 32 chunks; 0 for F32 inputs, which
 *            always run the single-pass form and ignore the workspace). The
 *            contents need no initialisation and are garbage afterwards; calls
 *            that share a workspace must be ordered on one stream.
 * Supported: dk = dv = 128, H >= 1, in_dtype F32 or BF16.
 * Value range (BF16 inputs): the value side of the chunk form (v, the states,
 *            the corrected writes u_r = beta_r (v_r - S'^T k_r) and the
 *            products formed from them) runs on float16 matrix operands, so
 *            every such entry must stay below 65,504 in magnitude (values of
 *            order one in the model; a larger one overflows to inf in o and
 *            the state). F32 inputs and the decode entry points have no such
 *            limit (float32 arithmetic throughout).
 * ---------------------------------------------------------------------- */
int kda_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                float scale, float lower_bound, const float* initial_state, float* final_state,
                void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                void* hip_stream);

size_t kda_prefill_workspace_bytes(int64_t num_tokens, int num_seqs, int H, int dk, int dv,
                                   kda_dtype in_dtype);

/* ------------------------------------------------------------------------
 * kda_prefill_noalloc -- kda_prefill without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Every argument keeps its meaning in kda_prefill; there is no workspace
 * argument. BF16 inputs run the two-pass form in a device-resident scratch
 * array of kda_prefill_noalloc_scratch_bytes() bytes (160 MiB), defined in the
 * library and held by each GPU the library runs on until the process ends;
 * its address is looked up once per device, on the first call with that
 * device current. F32 inputs run the single-pass form, which needs no scratch.
 * The call allocates nothing. A problem whose minimum workspace (one chunk slot
 * of 72,192 bytes plus a 64 KiB state carry per (sequence, head) unit, or a
 * slot for every chunk if that is less) exceeds the scratch is rejected with
 * KDA_ERR_WORKSPACE before anything is launched (at most 1,218 units, e.g. 19
 * sequences of 64 heads); below that, the chunks run in windows of as many
 * as the scratch holds (32-chunk windows at 64 heads). The scratch needs no
 * initialisation and keeps the last call's garbage. All calls on one GPU share it: calls that
 * overlap in time on one GPU (another stream, another host thread) race and
 * must be ordered by the caller.
 * ---------------------------------------------------------------------- */
int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                        float scale, float lower_bound, const float* initial_state, float* final_state,
                        void* o, kda_dtype out_dtype, void* hip_stream);

size_t kda_prefill_noalloc_scratch_bytes(void);

/* ----------------------------------------------------------------------
 * kda_prefill_gated -- kda_prefill with the gate prologue inside it.
 *
 * The decay and write strength come from the token mixer's projection rows,
 * as kda_gate_prologue forms them ("Ling-3.1-flash: a 560B hybrid-attention
 * MoE, counted from its safetensors headers", section "How KDA and MLA split
 * the work"): g = max(-exp(A_log[h]) softplus(f), lower_bound) per channel and
 * beta = sigmoid(b) per head, each rounded to bfloat16 as that prologue stores
 * them, so o and final_state equal kda_gate_prologue followed by kda_prefill
 * bit for bit. g and beta are formed in registers by the chunk-local pass and
 * never stored.
 *
 * f          bfloat16 rows [num_tokens, >= H*dk], row stride f_ld elements (a
 *            multiple of 8 below 2^24), 16-byte aligned; channel h*dk + c of a
 *            row is channel c of head h.
 * b          bfloat16 rows [num_tokens, >= H], row stride b_ld (below 2^24).
 * A_log      float32 [H].
 * Everything else as kda_prefill; in_dtype must be BF16 and a workspace is
 * required (the two-pass form: KDA_ERR_UNSUPPORTED / KDA_ERR_WORKSPACE
 * otherwise). f and b may overlap each other and q, k, v (they are read
 * only), not o, final_state or the workspace.
 * ---------------------------------------------------------------------- */
int kda_prefill_gated(const void* q, const void* k, const void* v, const void* f, int64_t f_ld, const void* b,
                      int64_t b_ld, const float* A_log, kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                      const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                      float scale, float lower_bound, const float* initial_state, float* final_state,
                      void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_prefill_snapshots -- kda_prefill that also saves the state at fixed
 * token positions of every sequence.
 *
 * A recurrent state summarises everything before it, so a cached prefix can
 * only be resumed where a state was saved; engines line these checkpoints up
 * with their cache blocks ("Ling-3.1-flash: What 63 Linear-Attention Layers Do
 * to the KV Budget", section "Where the hybrid makes serving harder").
 *
 * Every argument of kda_prefill keeps its meaning, plus:
 * snapshot_interval  tokens between snapshots, a positive multiple of 64.
 * snapshot_slots     snapshots per sequence that `snapshots` has room for:
 *            at least floor(L / snapshot_interval) for the longest sequence
 *            length L (else KDA_ERR_INVALID_ARG).
 * snapshots  float32 [num_seqs, snapshot_slots, H, dk, dv], caller-owned.
 *            snapshots[n][j] = the state of sequence n after its first
 *            (j + 1) * snapshot_interval tokens (starting from its initial
 *            state), for j < floor(L_n / snapshot_interval); other slots are
 *            not written. Must not overlap any other tensor.
 * ---------------------------------------------------------------------- */
int kda_prefill_snapshots(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                          const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                          float scale, float lower_bound, const float* initial_state, float* final_state,
                          void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          int64_t snapshot_interval, int64_t snapshot_slots, float* snapshots,
                          void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_prefill_segment_maps -- the affine map of every segment on the state.
 *
 * A prefill can be cut along the sequence only if the recurrent state can be
 * handed across the cuts; the engine the pages describe leaves prefill context
 * parallelism off for this mixer because it lacks that state handling
 * ("Ling-3.1-flash: What 63 Linear-Attention Layers Do to the KV Budget",
 * section "Where the hybrid makes serving harder"). The update of "Ling-3.1-
 * flash: Grouped Routing and Two Different MLA Caches", section "KDA replaces a
 * token list with a recurrent matrix", is linear in the state, so a segment of
 * tokens maps a start state S_in to S_out = M S_in + N with
 *   M = A_T ... A_1,  A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)  (dk x dk),
 *   N = the state after the segment from a zero state             (dk x dv).
 * Every segment's (M, N) is computed at once without knowing the states
 * before it; kda_affine_apply then chains them and kda_prefill (with those
 * initial states) forms each segment's outputs.
 *
 * Arguments as kda_prefill (each sequence of cu_seqlens is a segment), less q,
 * o and the states, plus:
 * M_out  float32 [num_seqs, H, dk, dk], caller-owned; an empty segment gives I.
 * N_out  float32 [num_seqs, H, dk, dv], caller-owned; an empty segment gives 0.
 *        Neither may overlap the other, an input or the workspace.
 * Supported: in_dtype BF16 only (the two-pass form; a workspace is required,
 * sized as for kda_prefill), dk = dv = 128.
 * ---------------------------------------------------------------------- */
int kda_prefill_segment_maps(const void* k, const void* v, const void* g, const void* beta, kda_dtype in_dtype,
                             int64_t num_tokens, int H, int dk, int dv,
                             const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                             float lower_bound, float* M_out, float* N_out, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_affine_apply -- Y[b] = M[b] X[b] (+ N[b]) for b < count.
 *
 * Applies segment maps (kda_prefill_segment_maps) to states, and composes
 * maps: (M2, N2) after (M1, N1) is (M2 M1, M2 N1 + N2), two calls.
 * M float32 [count, dk, dk]; X, N, Y float32 [count, dk, dv]; N may be NULL
 * (no addition). Y must not overlap M or X; it may be N itself (exactly).
 * float32 arithmetic, accumulation in a fixed order (deterministic).
 * Supported: dk = dv = 128; count = 0 does nothing.
 * ---------------------------------------------------------------------- */
int kda_affine_apply(const float* M, const float* X, const float* N, float* Y, int64_t count, int dk, int dv,
                     void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_decode_step -- one new token for each of B sequences, state in place.
 *
 * The same recurrence with T = 1 (retention, corrected write, read after the
 * write), as in "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches",
 * section "KDA replaces a token list with a recurrent matrix". Each step reads
 * and writes every sequence's [H, dk, dv] float32 state exactly once.
 *
 * q, k, g [B, H, dk], v [B, H, dv], beta [B, H]: in_dtype.
 * state   float32 [B, H, dk, dv], read and overwritten with the new state
 *         (kda_decode_multi with num_tokens = 1 takes a bfloat16 state too).
 * o       [B, H, dv] out_dtype.
 * lower_bound  log-retention floor (-5 in the model): any value <= 0, -inf
 *         included (no clamp); NaN or a positive floor returns
 *         KDA_ERR_INVALID_ARG.
 * Supported: dk = dv = 128, B >= 1, H >= 1.
 * ---------------------------------------------------------------------- */
int kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    kda_dtype in_dtype, int B, int H, int dk, int dv, float scale,
                    float lower_bound, float* state, void* o, kda_dtype out_dtype,
                    void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_decode_multi -- num_tokens new tokens for each of B sequences in one
 * pass over the state (the draft tokens of speculative decoding, to verify),
 * with the state stored in float32 or bfloat16.
 *
 * The recurrence applied token by token, as in kda_decode_step. A multi-token
 * prediction layer serves as the draft head, and about 2.1 to 2.6 tokens are
 * accepted per step ("Ling-3.1-flash: What 63 Linear-Attention Layers Do to
 * the KV Budget", section "Fitting it on a node"); rejected tokens must not
 * leave their writes in the state, hence the per-token states. The same page
 * (section "The memory math") puts the state at 252 MiB per sequence in FP32
 * and 126 MiB in BF16; with state_dtype BF16 the state is read into float32,
 * updated in float32 and rounded to bfloat16 (nearest even) when stored, which
 * halves the bytes of a decode step. num_tokens = 1 is a plain decode step.
 *
 * q, k, g [B, num_tokens, H, dk], v [B, num_tokens, H, dv],
 * beta [B, num_tokens, H]: in_dtype.
 * state   [B, H, dk, dv] in state_dtype, the state before the first token.
 *         With token_states NULL it is overwritten with the state after the
 *         last token; otherwise it is only read.
 * token_states  [B, num_tokens, H, dk, dv] in state_dtype or NULL: entry
 *         [b][t] = the state after token t of sequence b. Must not overlap
 *         another tensor.
 * o       [B, num_tokens, H, dv] out_dtype.
 * Supported: dk = dv = 128, B, H, num_tokens >= 1.
 * ---------------------------------------------------------------------- */
int kda_decode_multi(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     kda_dtype in_dtype, int B, int num_tokens, int H, int dk, int dv, float scale,
                     float lower_bound, void* state, void* token_states, kda_dtype state_dtype, void* o,
                     kda_dtype out_dtype, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_decode_commit -- keep the state of the accepted draft prefix.
 *
 * After verification, sequence b has accepted[b] of its num_tokens draft
 * tokens (same page and section as kda_decode_multi): its state becomes the
 * state after its last accepted token.
 *
 * token_states  [B, num_tokens, H, dk, dv] in state_dtype, from
 *               kda_decode_multi.
 * accepted      int32 [B], device. 1 <= accepted[b] <= num_tokens:
 *               state[b] = token_states[b][accepted[b] - 1] (a copy); any
 *               other value leaves state[b] as it is.
 * state         [B, H, dk, dv] in state_dtype, must not overlap token_states.
 * Supported: dk = dv = 128.
 * ---------------------------------------------------------------------- */
int kda_decode_commit(const void* token_states, const int32_t* accepted, int B, int num_tokens, int H, int dk,
                      int dv, void* state, kda_dtype state_dtype, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_state_convert -- states between float32 and bfloat16 storage.
 *
 * The state may be held in BF16 between decode steps ("Ling-3.1-flash: What
 * 63 Linear-Attention Layers Do to the KV Budget", section "The memory math");
 * prefill produces float32 states, converted once with this call.
 * dst[i] = src[i] for i < count, rounded to nearest even when narrowing
 * (same dtypes: a copy). src and dst must not overlap.
 * ---------------------------------------------------------------------- */
int kda_state_convert(const void* src, kda_dtype src_dtype, void* dst, kda_dtype dst_dtype, int64_t count,
                      void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_gemv_fp8 -- y = x W^T for a few rows x, with W in block FP8.
 *
 * The release stores its dense weights as FP8 E4M3 in 128 x 128 blocks with
 * one float32 scale per block ("Ling-3.1-flash: Grouped Routing and Two
 * Different MLA Caches", section "Production boundaries"; "Ling-3.1-flash: a
 * 560B hybrid-attention MoE, counted from its safetensors headers", section
 * "What is in the files"), and a batch-1 decode step is mostly the reading of
 * those weights (same page, "What the cut does not buy"); an FP8 block GEMV is
 * among the Hopper decode settings ("Ling-3.1-flash: What 63 Linear-Attention
 * Layers Do to the KV Budget", section "Fitting it on a node"). E4M3 is the
 * OCP FP8 format (bias 7, no infinities, 0x7F/0xFF NaN, largest 448).
 *
 * x        bfloat16 [M, K], row stride ldx (a multiple of 8), 1 <= M <= 8.
 * w        E4M3 codes [N, K], row stride ldw (bytes, a multiple of 16).
 * w_scale  float32 [ceil(N/128), K/128], row stride ws_ld:
 *          W[n, k] = e4m3(w[n, k]) * w_scale[n/128, k/128].
 * y        [M, N] y_dtype, row stride ldy; y[m, n] = sum_k x[m, k] W[n, k]
 *          (float32 accumulation). K must be a multiple of 128.
 * ---------------------------------------------------------------------- */
int kda_gemv_fp8(const void* x, int64_t ldx, const uint8_t* w, int64_t ldw, const float* w_scale, int64_t ws_ld,
                 void* y, int64_t ldy, int M, int64_t N, int64_t K, kda_dtype x_dtype, kda_dtype y_dtype,
                 void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_output_norm_gate_fp8 -- the epilogue with its output quantized to FP8.
 *
 * As kda_output_norm_gate (per-head RMSNorm x weight x sigmoid(gate)), with
 * the output quantized dynamically for an FP8 output projection (the pages
 * name block FP8 weights with dynamic activation quantization, section
 * "Production boundaries" above, and a fused KDA output quantization among
 * the Hopper decode settings: "Ling-3.1-flash: What 63 Linear-Attention Layers
 * Do to the KV Budget", section "Fitting it on a node"). One group per
 * (token, head) = 128 channels: scale = amax / 448 (1 for an all-zero group),
 * code = E4M3 of y / scale, rounded to nearest even.
 *
 * o        [num_tokens, H, dv] o_dtype.  gate: [num_tokens, >= H*dv]
 *          gate_dtype, row stride gate_ld (a multiple of 8).
 * y_codes  uint8 [num_tokens, H*dv]; y_scales float32 [num_tokens, H].
 * Supported: dv = 128.
 * ---------------------------------------------------------------------- */
int kda_output_norm_gate_fp8(const void* o, kda_dtype o_dtype, const void* gate, int64_t gate_ld,
                             kda_dtype gate_dtype, const float* norm_weight, int64_t num_tokens, int H, int dv,
                             float eps, uint8_t* y_codes, float* y_scales, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_quantize_fp8 -- dynamic activation quantization to block FP8.
 *
 * The pages pair block-FP8 E4M3 weights (128 x 128 scale blocks) with a
 * dynamic quantization of the activations ("Ling-3.1-flash: Grouped Routing
 * and Two Different MLA Caches", section "Production boundaries"). Here each
 * row is quantized in groups of 128 consecutive columns, each group with its
 * own float32 scale, so that X W^T can run on FP8 operands (kda_gemm_fp8).
 * Every rounding decision is taken in float32: scale = amax / 448 (1 for an
 * all-zero group), q = x / scale (correctly rounded division), clamped to
 * +-448, code = E4M3 nearest to q, ties to even.
 *
 * x       [M, K] x_dtype (float32 or bfloat16), row stride ldx (a multiple
 *         of 8), 16-byte aligned; finite values.
 * codes   uint8 [M, K] E4M3, row stride ldc (a multiple of 8), 8-byte aligned.
 * scales  float32 [M, K/128], row stride ld_scale.
 * K must be a multiple of 128. Outputs may not overlap each other or x.
 * ---------------------------------------------------------------------- */
int kda_quantize_fp8(const void* x, int64_t ldx, kda_dtype x_dtype, int64_t M, int64_t K, uint8_t* codes,
                     int64_t ldc, float* scales, int64_t ld_scale, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_gemm_fp8 -- Y = X W^T with both operands block FP8 (W8A8).
 *
 * The projection form of the pages' block-FP8 scheme (section "Production
 * boundaries" above; the Hopper decode settings list an FP8 block GEMV,
 * "Ling-3.1-flash: What 63 Linear-Attention Layers Do to the KV Budget",
 * section "Fitting it on a node"):
 *   X[m, k] = e4m3(x[m, k]) * x_scale[m, k/128]      (as kda_quantize_fp8 or
 *                                                     kda_output_norm_gate_fp8 write them)
 *   W[n, k] = e4m3(w[n, k]) * w_scale[n/128, k/128]  (128 x 128 blocks)
 *   Y[m, n] = sum_k X[m, k] W[n, k]: each 128-column block's sum of E4M3
 *             products is scaled once and the blocks are added in float32.
 *             M <= 8 forms the block sums in float32 as well; the matrix-core
 *             form's FP8 instruction forms them with about 14 bits of
 *             relative precision (the product of a block then differs from
 *             the exact one by ~1e-4 of the output's magnitude).
 *
 * x        uint8 [M, K], row stride ldx (a multiple of 16), 16-byte aligned.
 * x_scale  float32 [M, K/128], row stride xs_ld.
 * w        uint8 [N, K], row stride ldw (a multiple of 16), 16-byte aligned.
 * w_scale  float32 [ceil(N/128), K/128], row stride ws_ld.
 * y        [M, N] y_dtype (float32 or bfloat16, rounded to nearest even), row
 *          stride ldy; may not overlap an input.
 * K must be a multiple of 128. M <= 8 runs the weight-streaming GEMV forms of
 * kda_gemv_fp8 (decode); larger M the matrix-core GEMM (prefill).
 * ---------------------------------------------------------------------- */
int kda_gemm_fp8(const uint8_t* x, int64_t ldx, const float* x_scale, int64_t xs_ld, const uint8_t* w, int64_t ldw,
                 const float* w_scale, int64_t ws_ld, void* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                 kda_dtype y_dtype, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_conv_state_update -- decode-time causal short convolution.
 *
 * One causal depthwise convolution of width W (4 in the model) per projection
 * stream, followed by SiLU ("Ling-3.1-flash: Grouped Routing and Two Different
 * MLA Caches", section "KDA replaces a token list with a recurrent matrix";
 * the convolution tails are counted in "Ling-3.1-flash: What 63 Linear-
 * Attention Layers Do to the KV Budget", section "The memory math").
 *
 * x          B rows of C     new input token per sequence, row b at x + b * x_ld
 * conv_state [B, W-1, C]     the previous W-1 inputs, oldest first; updated in
 *                            place to the last W-1 inputs (shift left, append x)
 * weight     [C, W]          weight[:, W-1] multiplies the current input
 * bias       [C] or NULL
 * y          [B, C]          y = act(sum_j weight[c, j] * window[j] + bias[c]),
 *                            act = SiLU if apply_silu else identity, then, if
 *                            l2norm_group = 128, each group of 128 channels is
 *                            scaled by 1 / sqrt(sum(y^2) + l2norm_eps) (the
 *                            per-head q/k normalisation of the same section).
 * All in `dtype`. y must not overlap x or conv_state; conv_state must not
 * overlap x. The kept history is copied bit for bit. Supported: 2 <= W <= 8,
 * C a multiple of 128, l2norm_group 0 or 128.
 * ---------------------------------------------------------------------- */
int kda_conv_state_update(const void* x, int64_t x_ld, void* conv_state, const void* weight, const void* bias,
                          kda_dtype dtype, int B, int C, int W, int apply_silu,
                          int l2norm_group, float l2norm_eps, void* y, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_conv_prefill -- the prologue convolution over packed sequences.
 *
 * Causal depthwise convolution of width W per sequence (no leakage across
 * cu_seqlens boundaries), optional SiLU, then optional L2 normalisation over
 * each group of `l2norm_group` channels (the per-head q/k normalisation of the
 * same flozi.net section): y <- y / sqrt(sum(y^2) + l2norm_eps).
 *
 * x           rows of C channels, row r at x + r * x_ld (in_dtype = dtype)
 * cu_seqlens_*  as for kda_prefill
 * weight [C, W], bias [C] or NULL
 * conv_state_in  [num_seqs, W-1, C] history before each sequence, or NULL (zeros)
 * conv_state_out [num_seqs, W-1, C] last W-1 inputs of each sequence (taking
 *             history into account for short sequences), or NULL. Must not
 *             overlap conv_state_in.
 * l2norm_group  0 (off) or 128 (per-head normalisation); C a multiple of 128
 * y           rows of C channels at y + r * y_ld; must not overlap x
 * ---------------------------------------------------------------------- */
int kda_conv_prefill(const void* x, int64_t x_ld, int64_t num_tokens, int C, int W,
                     const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                     const void* weight, const void* bias, const void* conv_state_in,
                     void* conv_state_out, int apply_silu, int l2norm_group, float l2norm_eps,
                     void* y, int64_t y_ld, kda_dtype dtype, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_gate_prologue -- log-retention and write strength from projections.
 *
 * "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its safetensors
 * headers", section "How KDA and MLA split the work": the per-channel decay
 * comes from f_proj and A_log, the write strength from b_proj (one scalar per
 * head). Here
 *   g    = max(-exp(A_log[h]) * softplus(f), lower_bound)      [T, H, dk]
 *   beta = sigmoid(b)                                            [T, H]
 * f rows of H*dk at f + t * f_ld; b rows of H at b + t * b_ld (in_dtype);
 * A_log float32 [H]; g_out [T, H, dk] and beta_out [T, H] in out_dtype.
 * lower_bound <= 0 and not NaN (else KDA_ERR_INVALID_ARG).
 * ---------------------------------------------------------------------- */
int kda_gate_prologue(const void* f, int64_t f_ld, const void* b, int64_t b_ld,
                      const float* A_log, int64_t num_tokens, int H, int dk, float lower_bound,
                      kda_dtype in_dtype, void* g_out, void* beta_out, kda_dtype out_dtype,
                      void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_output_norm_gate -- epilogue: per-head RMSNorm times sigmoid gate.
 *
 * The mixer normalises its output and multiplies it by a sigmoid gate before
 * the projection back to the hidden width of 4,096 (flozi.net page, section
 * "KDA replaces a token list with a recurrent matrix"). Per token and head:
 *   y = o / sqrt(mean(o^2) + eps) * norm_weight * sigmoid(gate)
 * o [T, H, dv] (o_dtype); gate rows of H*dv at gate + t * gate_ld (stored in
 * y_dtype); norm_weight float32 [dv]; y [T, H*dv] (y_dtype), must not overlap o.
 * ---------------------------------------------------------------------- */
int kda_output_norm_gate(const void* o, kda_dtype o_dtype, const void* gate, int64_t gate_ld,
                         const float* norm_weight, int64_t num_tokens, int H, int dv, float eps,
                         void* y, kda_dtype y_dtype, void* hip_stream);

/* ------------------------------------------------------------------------
 * kda_gemm -- C[M, N] = A[M, K] * B[N, K]^T on MFMA, float32 accumulation.
 *
 * The layer's dense projections: q, k, v, decay and gate are 4096 -> 8192,
 * the output projection 8192 -> 4096 ("Ling-3.1-flash: a 560B hybrid-attention
 * MoE ...", section "How KDA and MLA split the work": six 8192 x 4096 matrices
 * per KDA layer). Weights are stored [out, in].
 * A rows at A + m * lda, B rows at B + n * ldb (ab_dtype = KDA_BF16),
 * C rows at C + m * ldc (c_dtype). K must be a multiple of 8; lda, ldb
 * multiples of 8, ldc a multiple of 4. C must not overlap A or B.
 * ---------------------------------------------------------------------- */
int kda_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, kda_dtype ab_dtype, kda_dtype c_dtype,
             void* hip_stream);

/* ------------------------------------------------------------------------
 * Size helpers. kda_state_bytes(64, 128, 128, KDA_F32) = 4,194,304: one
 * [64,128,128] FP32 matrix per layer, 252 MiB over 63 layers (flozi.net page,
 * section "KDA replaces a token list with a recurrent matrix").
 * kda_conv_state_bytes(3, 4, 8192, KDA_BF16) = 147,456 bytes per layer for
 * the q/k/v convolution tails (width-4 convolution of "Ling-3.1-flash: What
 * 63 Linear-Attention Layers Do to the KV Budget", section "The memory math").
 * Both return 0 for non-positive sizes.
 * ---------------------------------------------------------------------- */
size_t kda_state_bytes(int H, int dk, int dv, kda_dtype dtype);
size_t kda_conv_state_bytes(int streams, int W, int C, kda_dtype dtype);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kda_last_error(void);

/* KDA_VERSION of the built library. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
