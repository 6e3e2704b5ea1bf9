// kda_internal.h -- argument blocks and launchers shared by the host API and
// the kernel translation units. Host validation happens in kda_api.cpp before
// any launcher is called; launchers assume valid arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum DType : int { F32 = 0, BF16 = 1 };

// Tq tokens per sequence (1 for a plain decode step); inputs [B, Tq, H, d];
// states in state_dtype (float32 or bfloat16 storage, float32 arithmetic)
struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    void* state;         // [B, H, 128, 128]: written in place unless token_states is set
    void* token_states;  // [B, Tq, H, 128, 128] (state after each token) or null
    void* o;
    int B, H, Tq;
    float scale, lower_bound;
    DType in_dtype, out_dtype, state_dtype;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// state[b] <- token_states[b][accepted[b] - 1] for 1 <= accepted[b] <= Tq
hipError_t launch_decode_commit(const void* token_states, const int32_t* accepted, void* state, int B, int Tq, int H,
                                DType state_dtype, hipStream_t s);
// dst[i] = src[i] converted (float32 <-> bfloat16, round to nearest even)
hipError_t launch_convert(const void* src, DType src_dtype, void* dst, DType dst_dtype, int64_t n, hipStream_t s);

struct ConvUpdateArgs {
    const void* x;
    int64_t x_ld;
    void* conv_state;
    const void *weight, *bias;
    void* y;
    int B, C, W, apply_silu, l2_group;
    float l2_eps;
    DType dtype;
};
hipError_t launch_conv_update(const ConvUpdateArgs& a, hipStream_t s);

struct ConvPrefillArgs {
    const void* x;
    int64_t x_ld, y_ld, num_tokens;
    int C, W, num_seqs, apply_silu, l2_group;
    int64_t seq_len;  // used when cu_seqlens is null: equal-length sequences
    const int32_t* cu_seqlens;
    const void *weight, *bias, *state_in;
    void *state_out, *y;
    float l2_eps;
    DType dtype;
};
hipError_t launch_conv_prefill(const ConvPrefillArgs& a, hipStream_t s);

struct GateArgs {
    const void *f, *b;
    int64_t f_ld, b_ld, num_tokens;
    const float* A_log;
    void *g_out, *beta_out;
    int H, dk;
    float lower_bound;
    DType in_dtype, out_dtype;
};
hipError_t launch_gate(const GateArgs& a, hipStream_t s);

struct NormGateArgs {
    const void *o, *gate;
    int64_t gate_ld, num_tokens;
    const float* w;
    void* y;
    int H, dv;
    float eps;
    DType o_dtype, y_dtype;
};
hipError_t launch_norm_gate(const NormGateArgs& a, hipStream_t s);

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const int32_t* cu_seqlens;  // device, or null => equal lengths of seq_len
    int64_t seq_len;
    const float* s0;  // [N, H, 128, 128] or null
    float* sT;        // [N, H, 128, 128] or null
    void* o;
    int num_seqs, H;
    float scale, lower_bound;
    DType in_dtype, out_dtype;
    // state snapshots: after every snap_interval tokens of a sequence (a
    // multiple of 64), into snap[n][j] of [N, snap_slots, H, 128, 128]; off when null
    float* snap;
    int64_t snap_interval, snap_slots;
    // segment maps (two-pass form only): when set, the call computes for every
    // sequence the affine map S_out = M S_in + N of its tokens, M into map_M
    // [N, H, 128, 128] and N into sT, and writes no output (s0, o and snap unused)
    float* map_M;
    // gate prologue inside the prefill (two-pass form only): when gate_f is
    // set, g = max(-exp(A_log[h]) softplus(f), lower_bound) and beta =
    // sigmoid(b) are formed from the projection rows f [T, >= H*128] (row
    // stride gate_f_ld) and b [T, >= H] (gate_b_ld), each rounded to bfloat16
    // as the gate prologue stores them, in place of the g and beta inputs
    const void *gate_f, *gate_b;
    int64_t gate_f_ld, gate_b_ld;
    const float* A_log;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
// Two-pass form (bfloat16 inputs): per-chunk products in `ws`, then the state
// recurrence. max_chunks = the largest number of 64-token chunks of one
// sequence. ws_bytes must hold at least one chunk slot per (sequence, head),
// plus the float32 state carry when the slots cannot hold every chunk.
// cu_host: the host copy of cu_seqlens (null for equal lengths), from which
// each window's count of sequences still running sizes its launches.
hipError_t launch_prefill_split(const PrefillArgs& a, void* ws, size_t ws_bytes, int64_t max_chunks,
                                const int32_t* cu_host, hipStream_t s);
size_t prefill_split_slot_bytes();
// kda_prefill_noalloc: the two-pass workspace lives in a device array of this
// size (one per GPU, held until the process ends); prefill_static_scratch
// returns its address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)160 << 20;
hipError_t prefill_static_scratch(void** ptr);
// Y[b] = M[b] X[b] (+ N[b]) for b < count: float32 [count, 128, 128] matrices
hipError_t launch_affine_apply(const float* M, const float* X, const float* N, float* Y, int64_t count,
                               hipStream_t s);

// y[M, N] = x[M, K] W^T, W block-FP8: W[n, k] = e4m3(w[n, k]) * w_scale[n/128, k/128]
// With xs set, x holds E4M3 codes and X[m, k] = e4m3(x[m, k]) * xs[m, k/128]
// (activations quantized per row and 128-column group: W8A8).
struct Fp8GemvArgs {
    const void* x;        // bf16 [M, K] (xs null) or e4m3 codes [M, K], row stride ldx
    const uint8_t* w;     // e4m3 codes [N, K], row stride ldw
    const float* ws;      // [ceil(N/128), K/128], row stride ws_ld
    void* y;              // [M, N], row stride ldy
    int64_t ldx, ldw, ws_ld, ldy, N, K;
    int64_t M;
    DType y_dtype;
    const float* xs = nullptr;  // [M, K/128], row stride xs_ld
    int64_t xs_ld = 0;
};
hipError_t launch_gemv_fp8(const Fp8GemvArgs& a, hipStream_t s);

// W8A8 for many rows: y[M, N] = X W^T with X and W as above (xs required),
// on the FP8 matrix cores
hipError_t launch_gemm_fp8(const Fp8GemvArgs& a, hipStream_t s);

// dynamic activation quantization: per row and group of 128 columns,
// scale = amax / 448 (1 for an all-zero group), code = E4M3(x / scale)
struct QuantFp8Args {
    const void* x;
    uint8_t* codes;
    float* scales;
    int64_t ldx, ldc, lds, M, K;
    DType x_dtype;
};
hipError_t launch_quantize_fp8(const QuantFp8Args& a, hipStream_t s);

// the epilogue with its output quantized to e4m3 per (token, head)
struct NormGateFp8Args {
    const void *o, *gate;
    int64_t gate_ld, num_tokens;
    const float* w;
    uint8_t* codes;   // [T, H * 128]
    float* scales;    // [T, H]
    int H;
    float eps;
    DType o_dtype, gate_dtype;
};
hipError_t launch_norm_gate_fp8(const NormGateFp8Args& a, hipStream_t s);

struct GemmArgs {
    const void *A, *B;
    void* C;
    int64_t lda, ldb, ldc, M, N, K;
    DType c_dtype;
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

}  // namespace kda
