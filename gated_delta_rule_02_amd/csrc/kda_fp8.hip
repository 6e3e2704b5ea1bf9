// kda_fp8.hip -- block FP8 for the token mixer (gfx950).
//
// The release stores its dense weights as FP8 E4M3 in 128 x 128 blocks with
// one float32 scale per block, with activations quantized dynamically
// ("Ling-3.1-flash: Grouped Routing and Two Different MLA Caches", section
// "Production boundaries"; "Ling-3.1-flash: a 560B hybrid-attention MoE,
// counted from its safetensors headers", section "What is in the files"), and
// at batch 1 a decode step is mostly the reading of those dense weights, half
// of them the KDA projections (same page, "Counting the parameters" and "What
// the cut does not buy"). Two kernels:
//
// * gemv_fp8_kernel: y[M, N] = x[M, K] W^T for a few rows of x (decode), W
//   streamed once from HBM as E4M3 codes and decoded by the hardware
//   conversion (OCP E4M3 on gfx950), its block scale applied once per
//   16-value dot product. A wavefront owns a few rows of W; a lane takes 16
//   consecutive k of each (16-byte non-temporal loads), so one load
//   instruction covers 1 KiB of a row, and several such steps of every row
//   are loaded before any is used; the partial dot products are summed
//   across the wavefront at the end. Reading whole rows in 1-KiB pieces
//   matters: forms that fed the matrix cores directly (16 rows x 64 bytes per
//   load instruction) streamed W at only 3.5-4.2 TB/s.
// * norm_gate_fp8_kernel: the epilogue (per-head RMSNorm x weight x
//   sigmoid(gate)) with its output quantized per (token, head) -- one group
//   of 128 channels: scale = amax / 448, codes = round-to-nearest-even E4M3
//   of y / scale (the hardware conversion); one wavefront per (token, head).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;  // wavefronts per workgroup

// 16 E4M3 codes (4 dwords) -> 16 floats
__device__ __forceinline__ void decode16(const u32x4_t& u, float* f)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[d], false);
        const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[d], true);
        f[4 * d + 0] = lo.x;
        f[4 * d + 1] = lo.y;
        f[4 * d + 2] = hi.x;
        f[4 * d + 3] = hi.y;
    }
}

// R rows of W per wavefront; the codes of S 1-KiB steps of every row are
// loaded at once (a lane's 16 values of each), then used. The R rows lie in
// one 128-row block (R divides 128), so a step's block scale is one load.
template <typename TOUT, int M, int R, int S>
__global__ __launch_bounds__(kWaves * 64) void gemv_fp8_kernel(Fp8GemvArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n0 = ((int64_t)blockIdx.x * kWaves + wave) * R;
    if (n0 >= a.N) return;
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
    const float* srow = a.ws + (n0 >> 7) * a.ws_ld;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

    // K is a multiple of 128: a lane's 16 values are in range or not at all
    for (int64_t kc = 0; kc < a.K; kc += S * 1024) {
        u32x4_t u[S][R];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t k = kc + s * 1024 + 16 * lane;
                const int64_t n = n0 + r;
                u[s][r] = (n < a.N && k < a.K) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.w + n * a.ldw + k))
                                               : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int64_t k = kc + s * 1024 + 16 * lane;
            if (k < a.K) {
                const float sc = srow[k >> 7];
                float xv[M][16];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const bf16_t* xp = x + m * a.ldx + k;
                    const f32x4 x0 = ld4(xp), x1 = ld4(xp + 4), x2 = ld4(xp + 8), x3 = ld4(xp + 12);
                    const float t[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                         x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
                    for (int e = 0; e < 16; ++e) xv[m][e] = t[e];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float w[16];
                    decode16(u[s][r], w);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        float d = 0.f;
#pragma unroll
                        for (int e = 0; e < 16; ++e) d += w[e] * xv[m][e];
                        acc[r][m] += sc * d;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = wave_sum(acc[r][m]);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = n0 + r;
            if (n < a.N) {
#pragma unroll
                for (int m = 0; m < M; ++m) st(static_cast<TOUT*>(a.y) + m * a.ldy + n, acc[r][m]);
            }
        }
    }
}

constexpr int kNormRows = 4;  // (token, head) rows per workgroup, one wavefront each

template <typename TO, typename TG>
__global__ __launch_bounds__(kNormRows * 64) void norm_gate_fp8_kernel(NormGateFp8Args a)
{
    const int64_t row = (int64_t)blockIdx.x * kNormRows + (threadIdx.x >> 6);
    if (row >= a.num_tokens * a.H) return;
    const int lane = threadIdx.x & 63;
    const int64_t t = row / a.H;
    const int h = (int)(row % a.H);
    const int c = 2 * lane;  // dv == 128
    const f32x2 ov = ld2(static_cast<const TO*>(a.o) + row * 128 + c);
    const float ms = wave_sum(ov.x * ov.x + ov.y * ov.y) * (1.0f / 128.0f);
    const float r = rsqrtf(ms + a.eps);
    const f32x2 gv = ld2(static_cast<const TG*>(a.gate) + t * a.gate_ld + (int64_t)h * 128 + c);
    const float y0 = ov.x * r * a.w[c] * sigmoidf_(gv.x);
    const float y1 = ov.y * r * a.w[c + 1] * sigmoidf_(gv.y);
    const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0 / scale, y1 / scale, 0, false);
    *reinterpret_cast<uint16_t*>(a.codes + row * 128 + c) = (uint16_t)(packed & 0xffff);
    if (lane == 0) a.scales[row] = scale;
}

}  // namespace

template <int M, int R, int S>
void launch_gemv_rs(const Fp8GemvArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.N + kWaves * R - 1) / (kWaves * R))), block(kWaves * 64);
    if (a.y_dtype == F32) hipLaunchKernelGGL((gemv_fp8_kernel<float, M, R, S>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemv_fp8_kernel<bf16_t, M, R, S>), grid, block, 0, s, a);
}

hipError_t launch_gemv_fp8(const Fp8GemvArgs& a, hipStream_t s)
{
    // one token: 2 rows per wavefront, 4 KiB of each in flight (measured
    // 29.2 us on the 41,024 x 4,096 projection against 30.7 us for 4 rows x
    // 1 KiB); more tokens: 4 rows x 1 KiB, x's values then serve 4 rows
    switch (a.M) {
        case 1: launch_gemv_rs<1, 2, 4>(a, s); break;
        case 2: launch_gemv_rs<2, 4, 1>(a, s); break;
        case 3: launch_gemv_rs<3, 4, 1>(a, s); break;
        case 4: launch_gemv_rs<4, 4, 1>(a, s); break;
        case 5: launch_gemv_rs<5, 4, 1>(a, s); break;
        case 6: launch_gemv_rs<6, 4, 1>(a, s); break;
        case 7: launch_gemv_rs<7, 4, 1>(a, s); break;
        case 8: launch_gemv_rs<8, 4, 1>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_norm_gate_fp8(const NormGateFp8Args& a, hipStream_t s)
{
    const int64_t rows = a.num_tokens * a.H;
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + kNormRows - 1) / kNormRows)), block(kNormRows * 64);
    if (a.o_dtype == F32) {
        if (a.gate_dtype == F32) hipLaunchKernelGGL((norm_gate_fp8_kernel<float, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((norm_gate_fp8_kernel<float, bf16_t>), grid, block, 0, s, a);
    } else {
        if (a.gate_dtype == F32) hipLaunchKernelGGL((norm_gate_fp8_kernel<bf16_t, float>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((norm_gate_fp8_kernel<bf16_t, bf16_t>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
