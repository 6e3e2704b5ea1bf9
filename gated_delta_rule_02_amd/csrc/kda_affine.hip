// kda_affine.hip -- Y = M X (+ N) for batches of 128 x 128 float32 matrices.
//
// The state after a stretch of tokens is an affine function of the state
// before it: the per-token update of "Ling-3.1-flash: Grouped Routing and Two
// Different MLA Caches" (flozi.net), section "KDA replaces a token list with a
// recurrent matrix", is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} +
// beta_t k_t v_t^T, linear in S_{t-1}. A segment's map is S_out = M S_in + N.
// This kernel applies a map to a state (Y = M S + N) and composes two maps
// ((M2, N2) after (M1, N1) = (M2 M1, M2 N1 + N2): two calls), the steps that
// stitch segments of one sequence processed apart back together.
//
// One workgroup of 256 threads per 32 x 32 tile of one Y: the 32 rows of M and
// the 32 columns of X it needs are staged in LDS (row-padded), each thread
// accumulates four consecutive outputs of one row in float32, in a fixed
// order (deterministic).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int kTile = 32;
constexpr int kPad = 4;  // row padding of the staged tiles (float32 elements)

__global__ __launch_bounds__(256) void affine_kernel(const float* __restrict__ M, const float* __restrict__ X,
                                                     const float* N, float* Y)
{
    __shared__ __attribute__((aligned(16))) float Ms[kTile][D + kPad];  // rows r0.. of M
    __shared__ __attribute__((aligned(16))) float Xs[D][kTile + kPad];  // columns c0.. of X
    const int tid = threadIdx.x;
    const int tile = blockIdx.x & 15;
    const size_t b = blockIdx.x >> 4;
    const int r0 = (tile >> 2) * kTile, c0 = (tile & 3) * kTile;
    const float* Mb = M + b * D * D;
    const float* Xb = X + b * D * D;
    // stage: 32 x 128 of M and 128 x 32 of X, 16 bytes per thread and step
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;            // [32 rows][32 float4]
        const int r = e >> 5, c = (e & 31) * 4;
        *reinterpret_cast<f32x4*>(&Ms[r][c]) = *reinterpret_cast<const f32x4*>(Mb + (size_t)(r0 + r) * D + c);
        const int xr = e >> 3, xc = (e & 7) * 4;  // [128 rows][8 float4]
        *reinterpret_cast<f32x4*>(&Xs[xr][xc]) = *reinterpret_cast<const f32x4*>(Xb + (size_t)xr * D + c0 + xc);
    }
    __syncthreads();
    const int r = tid >> 3, c = (tid & 7) * 4;  // this thread's row and first column within the tile
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = 0; k < D; ++k) {
        const float m = Ms[r][k];
        const f32x4 x = *reinterpret_cast<const f32x4*>(&Xs[k][c]);
        acc[0] = fmaf(m, x[0], acc[0]);
        acc[1] = fmaf(m, x[1], acc[1]);
        acc[2] = fmaf(m, x[2], acc[2]);
        acc[3] = fmaf(m, x[3], acc[3]);
    }
    const size_t o = b * D * D + (size_t)(r0 + r) * D + c0 + c;
    if (N) acc += *reinterpret_cast<const f32x4*>(N + o);
    *reinterpret_cast<f32x4*>(Y + o) = acc;
}

}  // namespace

hipError_t launch_affine_apply(const float* M, const float* X, const float* N, float* Y, int64_t count, hipStream_t s)
{
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(affine_kernel, dim3((unsigned)(count * 16)), dim3(256), 0, s, M, X, N, Y);
    return hipGetLastError();
}

}  // namespace kda
