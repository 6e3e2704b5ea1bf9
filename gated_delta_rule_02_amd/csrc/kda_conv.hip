// kda_conv.hip -- causal depthwise short convolution (+SiLU, + per-group L2).
//
// "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches" (flozi.net),
// section "KDA replaces a token list with a recurrent matrix": each of the q,
// k and v projections passes through its own causal convolution of width four
// with SiLU; the same section has q and k normalised. Taps run oldest to
// newest: weight[c, W-1] multiplies the current token, weight[c, 0] the token
// W-1 steps back. Tokens before a sequence's first come from its conv state
// (oldest first) or are zero.
//
// Both kernels are memory-bound elementwise passes. The decode update: a
// wavefront owns one group of 128 channels (two per lane), so that the
// per-head L2 norm is a single wavefront reduction. The prefill: 16 bytes of
// channels per lane, the L2 norm a reduction over the lanes of one group.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kMaxW = 8;
constexpr int kGroup = 128;     // channels per wavefront
constexpr int kWaves = 4;       // wavefronts per workgroup

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
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}

// Finish one output pair: activation, optional L2 over the wavefront's group.
__device__ __forceinline__ f32x2 finish(f32x2 acc, int apply_silu, int l2, float eps)
{
    if (apply_silu) {
        acc.x = siluf_(acc.x);
        acc.y = siluf_(acc.y);
    }
    if (l2) {
        const float ss = wave_sum(acc.x * acc.x + acc.y * acc.y);
        const float r = rsqrtf(ss + eps);
        acc.x *= r;
        acc.y *= r;
    }
    return acc;
}

// ---------------------------------------------------------------- decode step
template <typename T>
__global__ __launch_bounds__(kWaves * 64) void conv_update_kernel(ConvUpdateArgs a)
{
    const int b = blockIdx.x;
    const int grp = blockIdx.y * kWaves + (threadIdx.x >> 6);
    if (grp * kGroup >= a.C) return;  // whole wavefront leaves together
    const int c = grp * kGroup + 2 * (threadIdx.x & 63);
    const int W = a.W;
    const T* x = static_cast<const T*>(a.x) + (size_t)b * a.x_ld;
    T* st = static_cast<T*>(a.conv_state) + (size_t)b * (W - 1) * a.C;
    const T* w = static_cast<const T*>(a.weight);

    // window[j] = input j steps after the oldest kept one; window[W-1] = new x
    f32x2 win[kMaxW];
    const f32x2 xn = ld2(x + c);
#pragma unroll
    for (int j = 0; j < kMaxW; ++j) {
        if (j < W - 1) win[j] = ld2(st + (size_t)j * a.C + c);
        else if (j == W - 1) win[j] = xn;
    }

    f32x2 acc = {0.f, 0.f};
    if (a.bias) acc = ld2(static_cast<const T*>(a.bias) + c);
#pragma unroll
    for (int j = 0; j < kMaxW; ++j)
        if (j < W) {
            acc.x += ld(w + (size_t)c * W + j) * win[j].x;
            acc.y += ld(w + (size_t)(c + 1) * W + j) * win[j].y;
        }
    acc = finish(acc, a.apply_silu, a.l2_group != 0, a.l2_eps);
    st2(static_cast<T*>(a.y) + (size_t)b * a.C + c, acc.x, acc.y);

    // shift the window left by one and append the new input (values are
    // exactly representable in T, so the stored bits are unchanged copies)
#pragma unroll
    for (int j = 0; j < kMaxW - 1; ++j)
        if (j < W - 1) st2(st + (size_t)j * a.C + c, win[j + 1].x, win[j + 1].y);
}

// Wide form (W fixed at compile time): a lane owns 8 consecutive channels, so
// that every access is 16 bytes (the input, each state row, the output, the
// lane's 8 x W weights); a 16-lane row of the wavefront covers one group of
// 128 channels, whose L2 norm is a 16-lane reduction.
// Two sequences per thread (the second B/2 rows on), so that the lane's
// weights serve both; streamed data goes around the caches (non-temporal).
template <typename T, int W>
__global__ __launch_bounds__(kWaves * 64) void conv_update_wide_kernel(ConvUpdateArgs a)
{
    using V = Vec16<T>;
    constexpr int NV = 8 / V::N;  // 16-byte vectors per 8 channels
    const int half = (a.B + 1) / 2;
    const int c = (blockIdx.y * kWaves + (threadIdx.x >> 6)) * 512 + 8 * (threadIdx.x & 63);
    const bool in = c < a.C;  // C is a multiple of 128: whole 16-lane groups are in or out
    float wv[8 * W], bv[8];
    if (in) {
        // weights of channels c .. c + 7: 8 W consecutive values
        const T* wp = static_cast<const T*>(a.weight) + (size_t)c * W;
#pragma unroll
        for (int v = 0; v < 8 * W / V::N; ++v) V::unpack(ld16(wp + v * V::N), &wv[v * V::N]);
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = 0.f;
        if (a.bias) {
#pragma unroll
            for (int v = 0; v < NV; ++v) V::unpack(ld16(static_cast<const T*>(a.bias) + c + v * V::N), &bv[v * V::N]);
        }
    }
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const int b = blockIdx.x + rep * half;
        if (b >= a.B) break;  // uniform over the workgroup
        const T* x = static_cast<const T*>(a.x) + (size_t)b * a.x_ld + c;
        T* st = static_cast<T*>(a.conv_state) + (size_t)b * (W - 1) * a.C + c;
        float win[W][8], acc[8];
        if (in) {
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const T* src = j < W - 1 ? st + (size_t)j * a.C : x;
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    V::unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + v * V::N)),
                              &win[j][v * V::N]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[e] = bv[e];
#pragma unroll
                for (int j = 0; j < W; ++j) acc[e] += wv[e * W + j] * win[j][e];
            }
            if (a.apply_silu) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = siluf_(acc[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        }
        if (a.l2_group) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += acc[e] * acc[e];
            const float r = rsqrtf(group_sum<16>(ss) + a.l2_eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= r;
        }
        if (in) {
            T* y = static_cast<T*>(a.y) + (size_t)b * a.C + c;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                __builtin_nontemporal_store(V::pack(&acc[v * V::N]), reinterpret_cast<u32x4_t*>(y + v * V::N));
            // shift the window left by one and append the new input (bit copies)
#pragma unroll
            for (int j = 0; j < W - 1; ++j)
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    __builtin_nontemporal_store(V::pack(&win[j + 1][v * V::N]),
                                                reinterpret_cast<u32x4_t*>(st + (size_t)j * a.C + v * V::N));
        }
    }
}

// ---------------------------------------------------------------- prefill
__device__ __forceinline__ int find_seq(const int32_t* cu, int num_seqs, int64_t t)
{
    // largest n with cu[n] <= t and cu[n+1] > t (skips empty sequences)
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// A lane owns 16 bytes of channels (8 bfloat16 or 4 float32) and walks the
// workgroup's tile of tokens in order, keeping the W-1 inputs before the
// current token in registers, so every input row is read once (plus W-1 rows
// of history at the tile start). The rows of the tile are loaded 8 at a time
// ahead of their use; the streamed rows and outputs carry the non-temporal
// hint (the layer's three convolutions read and write 805 MB, more than the
// last-level cache: 68 -> 63 us per call at T = 8192, C = 8192; 16 rows ahead
// lowered the occupancy and took 109 us). The current sequence (start s, end e) is tracked per
// workgroup; at a sequence start the window is refilled from that sequence's
// conv state, or with zeros.
constexpr int kConvTok = 32;  // tokens per workgroup
constexpr int kConvBatch = 8; // rows loaded ahead

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_prefill_kernel(ConvPrefillArgs a)
{
    using V = Vec16<T>;
    constexpr int N = V::N;          // channels per lane
    constexpr int GL = kGroup / N;   // lanes per 128-channel group
    const int c = (blockIdx.y * 256 + threadIdx.x) * N;
    if (c >= a.C) return;  // C is a multiple of 128: whole groups leave together
    const T* x = static_cast<const T*>(a.x);
    const T* w = static_cast<const T*>(a.weight);
    const T* sin = static_cast<const T*>(a.state_in);

    float wt[W][N];  // wt[j][i] = weight[c + i][j]
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = 0; j < W; ++j) wt[j][i] = ld(w + (size_t)(c + i) * W + j);
    float bias[N];
#pragma unroll
    for (int i = 0; i < N; ++i) bias[i] = a.bias ? ld(static_cast<const T*>(a.bias) + c + i) : 0.0f;

    const int64_t t0 = (int64_t)blockIdx.x * kConvTok;
    const int64_t t1 = min<int64_t>(t0 + kConvTok, a.num_tokens);
    int n;
    int64_t s, e;
    if (a.cu_seqlens) {
        n = find_seq(a.cu_seqlens, a.num_seqs, t0);
        s = a.cu_seqlens[n];
        e = a.cu_seqlens[n + 1];
    } else {
        n = (int)(t0 / a.seq_len);
        s = (int64_t)n * a.seq_len;
        e = s + a.seq_len;
    }
    // input at position p < s of sequence n: its conv state (oldest first) or 0
    auto history = [&](int64_t p, float* out) {
        if (sin) {
            V::unpack(ld16(sin + ((size_t)n * (W - 1) + (size_t)((W - 1) - (s - p))) * a.C + c), out);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) out[i] = 0.0f;
        }
    };
    float win[W - 1][N];  // win[j]: the input W-1-j positions before the current token
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
        const int64_t p = t0 - (W - 1) + j;
        if (p >= s) V::unpack(ld16(x + p * a.x_ld + c), win[j]);
        else history(p, win[j]);
    }

    T* y = static_cast<T*>(a.y);
    for (int64_t tb = t0; tb < t1; tb += kConvBatch) {
        u32x4_t raw[kConvBatch];
#pragma unroll
        for (int r = 0; r < kConvBatch; ++r)
            raw[r] = tb + r < t1 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + (tb + r) * a.x_ld + c))
                                  : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < kConvBatch; ++r) {
            const int64_t t = tb + r;
            if (t >= t1) break;
            if (t == e) {
                // the next non-empty sequence starts at t
                if (a.cu_seqlens) {
                    do { ++n; } while (a.cu_seqlens[n + 1] <= t);
                    s = a.cu_seqlens[n];
                    e = a.cu_seqlens[n + 1];
                } else {
                    ++n;
                    s = e;
                    e = s + a.seq_len;
                }
#pragma unroll
                for (int j = 0; j < W - 1; ++j) history(t - (W - 1) + j, win[j]);
            }
            float xv[N], acc[N];
            V::unpack(raw[r], xv);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                float v = bias[i];
#pragma unroll
                for (int j = 0; j < W - 1; ++j) v += wt[j][i] * win[j][i];
                acc[i] = v + wt[W - 1][i] * xv[i];
            }
#pragma unroll
            for (int j = 0; j < W - 1; ++j)
#pragma unroll
                for (int i = 0; i < N; ++i) win[j][i] = j + 1 < W - 1 ? win[j + 1][i] : xv[i];
            if (a.apply_silu) {
#pragma unroll
                for (int i = 0; i < N; ++i) acc[i] = siluf_(acc[i]);
            }
            if (a.l2_group) {
                float ss = 0.0f;
#pragma unroll
                for (int i = 0; i < N; ++i) ss += acc[i] * acc[i];
                const float rn = rsqrtf(group_sum<GL>(ss) + a.l2_eps);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[i] *= rn;
            }
            __builtin_nontemporal_store(V::pack(acc), reinterpret_cast<u32x4_t*>(y + t * a.y_ld + c));
        }
    }
}

// Bit copies of two consecutive elements.
__device__ __forceinline__ void copy2(float* d, const float* p) { *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void copy2(bf16_t* d, const bf16_t* p) { *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void zero2(float* d) { *reinterpret_cast<uint2*>(d) = make_uint2(0u, 0u); }
__device__ __forceinline__ void zero2(bf16_t* d) { *reinterpret_cast<uint32_t*>(d) = 0u; }

// Last W-1 inputs of each sequence (history included for short sequences).
template <typename T>
__global__ void conv_state_out_kernel(ConvPrefillArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over N*(W-1)*C/2
    const int W = a.W;
    const int64_t pairs = (int64_t)a.C / 2;
    const int64_t total = (int64_t)a.num_seqs * (W - 1) * pairs;
    if (idx >= total) return;
    const int c = (int)(idx % pairs) * 2;
    const int j = (int)((idx / pairs) % (W - 1));
    const int n = (int)(idx / (pairs * (W - 1)));
    int64_t s, e;
    if (a.cu_seqlens) {
        s = a.cu_seqlens[n];
        e = a.cu_seqlens[n + 1];
    } else {
        s = (int64_t)n * a.seq_len;
        e = s + a.seq_len;
    }
    const int64_t p = e - (W - 1) + j;  // position of the j-th kept input
    const T* x = static_cast<const T*>(a.x);
    const T* sin = static_cast<const T*>(a.state_in);
    T* so = static_cast<T*>(a.state_out) + ((size_t)n * (W - 1) + j) * a.C + c;
    if (p >= s)
        copy2(so, x + p * a.x_ld + c);
    else if (sin)
        copy2(so, sin + ((size_t)n * (W - 1) + (size_t)((W - 1) - (s - p))) * a.C + c);
    else
        zero2(so);
}

}  // namespace

hipError_t launch_conv_update(const ConvUpdateArgs& a, hipStream_t s)
{
    // the wide form: 8 channels per lane, 16-byte accesses (C is a multiple
    // of 128 and every row 16-byte aligned)
    {
        const dim3 grid((unsigned)((a.B + 1) / 2), (unsigned)((a.C + 512 * kWaves - 1) / (512 * kWaves))),
            block(kWaves * 64);
        switch (a.W) {
#define KDA_CONVU_W(WW)                                                                                    \
    case WW:                                                                                               \
        if (a.dtype == F32) hipLaunchKernelGGL((conv_update_wide_kernel<float, WW>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((conv_update_wide_kernel<bf16_t, WW>), grid, block, 0, s, a);            \
        return hipGetLastError();
            KDA_CONVU_W(2) KDA_CONVU_W(3) KDA_CONVU_W(4) KDA_CONVU_W(5) KDA_CONVU_W(6) KDA_CONVU_W(7) KDA_CONVU_W(8)
#undef KDA_CONVU_W
            default: break;
        }
    }
    dim3 grid((unsigned)a.B, (unsigned)((a.C + kGroup * kWaves - 1) / (kGroup * kWaves))), block(kWaves * 64);
    if (a.dtype == F32)
        hipLaunchKernelGGL(conv_update_kernel<float>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(conv_update_kernel<bf16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_conv_prefill(const ConvPrefillArgs& a, hipStream_t s)
{
    if (a.num_tokens > 0) {
        const int ch = a.dtype == F32 ? 256 * 4 : 256 * 8;  // channels per workgroup
        const dim3 grid((unsigned)((a.num_tokens + kConvTok - 1) / kConvTok), (unsigned)((a.C + ch - 1) / ch)),
            block(256);
        switch (a.W) {
#define KDA_CONV_W(WW)                                                                              \
    case WW:                                                                                        \
        if (a.dtype == F32) hipLaunchKernelGGL((conv_prefill_kernel<float, WW>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((conv_prefill_kernel<bf16_t, WW>), grid, block, 0, s, a);           \
        break;
            KDA_CONV_W(2) KDA_CONV_W(3) KDA_CONV_W(4) KDA_CONV_W(5) KDA_CONV_W(6) KDA_CONV_W(7) KDA_CONV_W(8)
#undef KDA_CONV_W
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.state_out) {
        const int64_t total = (int64_t)a.num_seqs * (a.W - 1) * (a.C / 2);
        dim3 grid((unsigned)((total + 255) / 256)), block(256);
        if (a.dtype == F32)
            hipLaunchKernelGGL(conv_state_out_kernel<float>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(conv_state_out_kernel<bf16_t>, grid, block, 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
