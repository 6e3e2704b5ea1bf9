// kda_gemm.hip -- C[M,N] = A[M,K] B[N,K]^T, bfloat16 inputs, float32 accumulate.
//
// The token mixer's dense projections ("Ling-3.1-flash: a 560B hybrid-attention
// MoE, counted from its safetensors headers", section "How KDA and MLA split the
// work": q, k, v, decay and gate 4096 -> 8192 and the output 8192 -> 4096, all
// full rank). Both operands are K-contiguous, which is exactly the layout the
// 16x16x32 bf16 MFMA consumes: each lane takes 8 consecutive K values of one
// row of A and one row of B.
//
// Tiling: 256 threads, a 128 x 128 tile of C per workgroup, wavefronts in a
// 2 x 2 arrangement each owning 64 x 64 (4 x 4 MFMA tiles), K steps of 32
// staged through double-buffered LDS with 16-byte global loads.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_LD = BK + 8;  // padded row (bf16 elements)
constexpr int kThreads = 256;

__device__ __forceinline__ f32x4 mma32_bf16(const uint4& a, const uint4& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <typename TC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM][LDS_LD];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN][LDS_LD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const bf16_t* A = static_cast<const bf16_t*>(a.A);
    const bf16_t* B = static_cast<const bf16_t*>(a.B);

    // global -> register staging: 2 x 16 B of A and of B per thread per K step
    uint4 ra[2], rb[2];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = tid + j * kThreads;  // 0..511
            const int row = idx >> 2, kc = (idx & 3) * 8;
            const int64_t gm = m0 + row, gn = n0 + row, gk = k0 + kc;
            ra[j] = (gm < a.M && gk < a.K) ? *reinterpret_cast<const uint4*>(A + gm * a.lda + gk) : make_uint4(0, 0, 0, 0);
            rb[j] = (gn < a.N && gk < a.K) ? *reinterpret_cast<const uint4*>(B + gn * a.ldb + gk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int idx = tid + j * kThreads;
            const int row = idx >> 2, kc = (idx & 3) * 8;
            *reinterpret_cast<uint4*>(&sA[buf][row][kc]) = ra[j];
            *reinterpret_cast<uint4*>(&sB[buf][row][kc]) = rb[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)((a.K + BK - 1) / BK);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
        uint4 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const uint4*>(&sA[buf][wm + 16 * i + m16][8 * q4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const uint4*>(&sB[buf][wn + 16 * j + m16][8 * q4]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mma32_bf16(fa[i], fb[j], acc[i][j]);
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    TC* Cp = static_cast<TC*>(a.C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn + 16 * j + m16;
            if (col >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm + 16 * i + 4 * q4 + e;
                if (row < a.M) st(Cp + row * a.ldc + col, acc[i][j][e]);
            }
        }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM)), block(kThreads);
    if (a.c_dtype == F32)
        hipLaunchKernelGGL(gemm_kernel<float>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gemm_kernel<bf16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
