// kda_elementwise.hip -- gate prologue and output-norm x sigmoid-gate epilogue.
//
// Gate: "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its
// safetensors headers", section "How KDA and MLA split the work": per-channel
// decay from the full-rank f_proj and A_log, write strength from b_proj (one
// scalar per head). The log-retention is g = -exp(A_log[h]) softplus(f),
// bounded below by the safe-forget-gate floor (-5) of "Ling-3.1-flash: Grouped
// Routing and Two Different MLA Caches", section "KDA replaces a token list with
// a recurrent matrix"; beta = sigmoid(b).
//
// Epilogue: the same flozi.net section puts an output normalisation and a
// sigmoid gate before the output projection; here a per-head RMSNorm over the
// 128 value channels, a per-channel weight and sigmoid(gate).
//
// Both are one wavefront per (token, head) row of 128 channels, two channels
// per lane: the RMS is one wavefront reduction, accesses are 4/8-byte per lane.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kRowsPerBlock = 4;

template <typename T>
__device__ __forceinline__ void st2(T* p, float a, float b);
template <>
__device__ __forceinline__ void st2<float>(float* p, float a, float b)
{
    *reinterpret_cast<f32x2*>(p) = f32x2{a, b};
}
template <>
__device__ __forceinline__ void st2<bf16_t>(bf16_t* p, float a, float b)
{
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kRowsPerBlock * 64) void gate_kernel(GateArgs a)
{
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);  // t * H + h
    if (row >= a.num_tokens * a.H) return;
    const int lane = threadIdx.x & 63;
    const int64_t t = row / a.H;
    const int h = (int)(row % a.H);
    const float rate = __expf(a.A_log[h]);
    const TI* f = static_cast<const TI*>(a.f) + t * a.f_ld + (int64_t)h * a.dk;
    TO* g = static_cast<TO*>(a.g_out) + row * a.dk;
    for (int c = 2 * lane; c < a.dk; c += 128) {
        const f32x2 fv = ld2(f + c);
        st2(g + c, fmaxf(-rate * softplusf_(fv.x), a.lower_bound),
            fmaxf(-rate * softplusf_(fv.y), a.lower_bound));
    }
    if (lane == 0) {
        const float bv = ld(static_cast<const TI*>(a.b) + t * a.b_ld + h);
        st(static_cast<TO*>(a.beta_out) + row, sigmoidf_(bv));
    }
}

template <typename TO_, typename TY>
__global__ __launch_bounds__(kRowsPerBlock * 64) void norm_gate_kernel(NormGateArgs a)
{
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= a.num_tokens * a.H) return;
    const int lane = threadIdx.x & 63;
    const int64_t t = row / a.H;
    const int h = (int)(row % a.H);
    const int c = 2 * lane;  // dv == 128
    const f32x2 ov = ld2(static_cast<const TO_*>(a.o) + row * a.dv + c);
    const float ms = wave_sum(ov.x * ov.x + ov.y * ov.y) * (1.0f / 128.0f);
    const float r = rsqrtf(ms + a.eps);
    const f32x2 gv = ld2(static_cast<const TY*>(a.gate) + t * a.gate_ld + (int64_t)h * a.dv + c);
    const float w0 = a.w[c], w1 = a.w[c + 1];
    st2(static_cast<TY*>(a.y) + row * a.dv + c, ov.x * r * w0 * sigmoidf_(gv.x),
        ov.y * r * w1 * sigmoidf_(gv.y));
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, hipStream_t s)
{
    const int64_t rows = a.num_tokens * a.H;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
    if (a.in_dtype == F32) {
        if (a.out_dtype == F32) hipLaunchKernelGGL((gate_kernel<float, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gate_kernel<float, bf16_t>), grid, block, 0, s, a);
    } else {
        if (a.out_dtype == F32) hipLaunchKernelGGL((gate_kernel<bf16_t, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gate_kernel<bf16_t, bf16_t>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_norm_gate(const NormGateArgs& a, hipStream_t s)
{
    const int64_t rows = a.num_tokens * a.H;
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
    if (a.o_dtype == F32) {
        if (a.y_dtype == F32) hipLaunchKernelGGL((norm_gate_kernel<float, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((norm_gate_kernel<float, bf16_t>), grid, block, 0, s, a);
    } else {
        if (a.y_dtype == F32) hipLaunchKernelGGL((norm_gate_kernel<bf16_t, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((norm_gate_kernel<bf16_t, bf16_t>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
