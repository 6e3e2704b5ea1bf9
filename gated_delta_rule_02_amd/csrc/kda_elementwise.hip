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
// Both are memory-bound passes with 16-byte accesses where the storage type
// allows (layout and lane mapping at each kernel).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Gate: a lane owns 8 consecutive channels (one head: dk = 128) of 8 tokens;
// the rows are loaded before any is computed, 16-byte accesses for bfloat16.
constexpr int kGateTok = 8;
constexpr int kGateCh = 256 * 8;  // channels per workgroup

// the gate's input rows are read once: non-temporal (measured on the layer at
// T = 8192: the gate and the prefill after it 525 -> 500 us; default loads
// filled the last-level cache with the f columns of the projection)
template <typename T>
__device__ __forceinline__ void ld8(const T* p, float* f)
{
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
    if constexpr (sizeof(T) == 2) {
        Vec16<bf16_t>::unpack(__builtin_nontemporal_load(q), f);
    } else {
        Vec16<float>::unpack(__builtin_nontemporal_load(q), f);
        Vec16<float>::unpack(__builtin_nontemporal_load(q + 1), f + 4);
    }
}
template <typename T>
__device__ __forceinline__ void st8(T* p, const float* f)
{
    if constexpr (sizeof(T) == 2) {
        st16(p, Vec16<bf16_t>::pack(f));
    } else {
        st16(p, Vec16<float>::pack(f));
        st16(p + 4, Vec16<float>::pack(f + 4));
    }
}

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gate_kernel(GateArgs a)
{
    const int64_t t0 = (int64_t)blockIdx.x * kGateTok;
    const int nt = (int)min<int64_t>(kGateTok, a.num_tokens - t0);
    if (blockIdx.y == 0) {
        // beta = sigmoid(b) for the workgroup's tokens
        for (int i = threadIdx.x; i < nt * a.H; i += 256) {
            const int64_t t = t0 + i / a.H;
            const int h = i % a.H;
            st(static_cast<TO*>(a.beta_out) + t * a.H + h, sigmoidf_(ld(static_cast<const TI*>(a.b) + t * a.b_ld + h)));
        }
    }
    const int cc = blockIdx.y * kGateCh + threadIdx.x * 8;  // channel in [0, H * dk)
    if (cc >= a.H * a.dk) return;
    const float rate = __expf(a.A_log[cc / a.dk]);
    const TI* f = static_cast<const TI*>(a.f) + t0 * a.f_ld + cc;
    TO* g = static_cast<TO*>(a.g_out) + t0 * (int64_t)a.H * a.dk + cc;
    float fv[kGateTok][8];
#pragma unroll
    for (int r = 0; r < kGateTok; ++r)
        if (r < nt) ld8(f + r * a.f_ld, fv[r]);
#pragma unroll
    for (int r = 0; r < kGateTok; ++r) {
        if (r >= nt) break;
        float gv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = fmaxf(-rate * softplus_hw(fv[r][i]), a.lower_bound);
        st8(g + r * (int64_t)a.H * a.dk, gv);
    }
}

// The epilogue reads o and the gate columns once: non-temporal, so that y,
// which the output projection reads next, stays in the last-level cache
// (measured at T = 8192: the epilogue and the output projection after it
// 625-634 -> 588-590 us; the epilogue alone unchanged)
template <typename T> __device__ __forceinline__ f32x4 ld4_nt(const T* p);
template <> __device__ __forceinline__ f32x4 ld4_nt<float>(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
template <> __device__ __forceinline__ f32x4 ld4_nt<bf16_t>(const bf16_t* p)
{
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 u = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}

// Epilogue: a lane owns 4 consecutive channels; 32 lanes cover one (token,
// head) row, so a wavefront handles two rows and the RMS is a 32-lane sum.
constexpr int kNormRowsPerBlock = 8;

template <typename TO_, typename TY>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateArgs a)
{
    const int64_t row = (int64_t)blockIdx.x * kNormRowsPerBlock + (threadIdx.x >> 5);  // t * H + h
    if (row >= a.num_tokens * a.H) return;  // whole 32-lane halves leave together
    const int c = 4 * (threadIdx.x & 31);   // dv == 128
    const int64_t t = row / a.H;
    const int h = (int)(row % a.H);
    const f32x4 ov = ld4_nt(static_cast<const TO_*>(a.o) + row * a.dv + c);
    const f32x4 gv = ld4_nt(static_cast<const TY*>(a.gate) + t * a.gate_ld + (int64_t)h * a.dv + c);
    const f32x4 wv = ld4(a.w + c);
    const float ms = group_sum<32>(ov.x * ov.x + ov.y * ov.y + ov.z * ov.z + ov.w * ov.w) * (1.0f / 128.0f);
    const float r = rsqrtf(ms + a.eps);
    st4(static_cast<TY*>(a.y) + row * a.dv + c,
        f32x4{ov.x * r * wv.x * sigmoidf_(gv.x), ov.y * r * wv.y * sigmoidf_(gv.y),
              ov.z * r * wv.z * sigmoidf_(gv.z), ov.w * r * wv.w * sigmoidf_(gv.w)});
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, hipStream_t s)
{
    if (a.num_tokens == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.num_tokens + kGateTok - 1) / kGateTok),
                    (unsigned)(((int64_t)a.H * a.dk + kGateCh - 1) / kGateCh)),
        block(256);
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
    const dim3 grid((unsigned)((rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock)), block(256);
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
