// kda_decode.hip -- KDA decode for a batch of sequences (gfx950): one token
// per sequence, or a few (draft tokens to verify), keeping the state in
// registers between them.
//
// Per (sequence, head) and token the step is the recurrence of
// "Ling-3.1-flash: Grouped Routing and Two Different MLA Caches" (flozi.net),
// section "KDA replaces a token list with a recurrent matrix":
//   S' = Diag(alpha) S,   u = beta (v - S'^T k),   S = S' + k u^T,
//   o  = scale S^T q = scale (S'^T q + u (k . q)).
// The 128 x 128 float32 state (64 KiB) is the only large operand, so the kernel
// is bound by HBM: it reads every state once into registers with 16-byte
// coalesced loads, reduces the two column sums S'^T k and S'^T q across the
// workgroup, and writes the state back once from the same registers.
//
// Workgroup = one (sequence, head); every thread owns 4 (8) rows and 16 bytes of
// each (4 float32 or 8 bfloat16 columns), so a wavefront moves 1 KiB of
// contiguous state per access: 1024 threads for a float32 state, 256 for a
// bfloat16 one. Measured on the 1 GiB float32 decode workload: 256 threads x
// 16 rows 410 us, 512 x 8 410 us, 1024 x 4 386 us (the in-place stream of
// the state is the whole cost; the wider workgroup keeps more of it in
// flight).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

#ifndef KDA_DECODE_NT
#define KDA_DECODE_NT 1
#endif
#if KDA_DECODE_NT
// the state is streamed exactly once per step: non-temporal accesses keep it
// from displacing the small per-step inputs in the caches
#define KDA_NT_LOAD(p) __builtin_nontemporal_load(p)
#define KDA_NT_STORE(v, p) __builtin_nontemporal_store(v, p)
#else
#define KDA_NT_LOAD(p) (*(p))
#define KDA_NT_STORE(v, p) (*(p) = (v))
#endif

constexpr int D = 128;
#ifndef KDA_DECODE_THREADS
#define KDA_DECODE_THREADS 1024
#endif

// Thread mapping per state storage: every thread moves 16 bytes per row it
// owns (4 float32 or 8 bfloat16 columns); a wavefront covers 1 KiB of
// contiguous state per access. float32: 1024 threads x 4 rows (the 64 KiB
// state of one (sequence, head)); bfloat16: 256 threads x 8 rows (32 KiB),
// small enough that five workgroups fit a compute unit and keep ~160 KiB of
// state in flight per unit (measured on the 512 MiB bf16 workload: 128, 256,
// 512 and 1024 threads ran 221, 209, 226 and 380 us).
template <typename TS> struct Map {
    static constexpr int kCols = 16 / (int)sizeof(TS);   // columns per thread
    static constexpr int kLanesPerRow = D / kCols;        // 32 or 16
    static constexpr int kThreads = (int)sizeof(TS) == 4 ? KDA_DECODE_THREADS : 256;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kRowGroups = kThreads / kLanesPerRow;
    static constexpr int kRowsPerThread = D / kRowGroups;
    static constexpr int kQuads = kCols / 4;              // f32x4 per row segment
};

// kCols consecutive state elements as floats (kQuads f32x4), streamed once per step
__device__ __forceinline__ void ld_state(const float* p, f32x4* v) { v[0] = KDA_NT_LOAD(reinterpret_cast<const f32x4*>(p)); }
__device__ __forceinline__ void ld_state(const bf16_t* p, f32x4* v)
{
    const u32x4_t u = KDA_NT_LOAD(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
    for (int h = 0; h < 2; ++h)
        v[h] = f32x4{__uint_as_float(u[2 * h] << 16), __uint_as_float(u[2 * h] & 0xffff0000u),
                     __uint_as_float(u[2 * h + 1] << 16), __uint_as_float(u[2 * h + 1] & 0xffff0000u)};
}
__device__ __forceinline__ void st_state(float* p, const f32x4* v) { KDA_NT_STORE(v[0], reinterpret_cast<f32x4*>(p)); }
__device__ __forceinline__ void st_state(bf16_t* p, const f32x4* v)
{
    u32x4_t u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        u[2 * h] = pack_bf16x2(v[h].x, v[h].y);
        u[2 * h + 1] = pack_bf16x2(v[h].z, v[h].w);
    }
    KDA_NT_STORE(u, reinterpret_cast<u32x4_t*>(p));
}

template <typename TIN, typename TOUT, typename TS>
__global__ __launch_bounds__(Map<TS>::kThreads) void decode_kernel(DecodeArgs a)
{
    using M = Map<TS>;
    constexpr int kWaves = M::kWaves, kRowGroups = M::kRowGroups, kRows = M::kRowsPerThread, kQ = M::kQuads;
    const int bh = blockIdx.x;  // b * H + h
    const int bseq = bh / a.H, h = bh - bseq * a.H;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;

    __shared__ float s_alpha[D], s_k[D], s_q[D];
    __shared__ float s_part[kWaves][2][D];  // per-wave partial column sums (S'^T k, S'^T q)
    __shared__ float s_u[D];
    __shared__ float s_kq[2];

    // Issue the state loads first: they are the long-latency stream. Thread t
    // owns columns kCols (t % kLanesPerRow) .. +kCols-1 of the rows
    // t / kLanesPerRow + kRowGroups i.
    const int cg = t % M::kLanesPerRow;
    const int rg = t / M::kLanesPerRow;
    const int c0 = M::kCols * cg;
    TS* Sp = static_cast<TS*>(a.state) + (size_t)bh * D * D;
    f32x4 s[kRows][kQ];
#pragma unroll
    for (int i = 0; i < kRows; ++i) ld_state(Sp + (size_t)(rg + kRowGroups * i) * D + c0, s[i]);

    // the Tq tokens of this sequence in order; the state stays in registers
    for (int tk = 0; tk < a.Tq; ++tk) {
        const size_t row = ((size_t)bseq * a.Tq + tk) * a.H + h;  // token row of [B, Tq, H, d]
        const TIN* q = static_cast<const TIN*>(a.q) + row * D;
        const TIN* k = static_cast<const TIN*>(a.k) + row * D;
        const TIN* g = static_cast<const TIN*>(a.g) + row * D;
        if (tk > 0) __syncthreads();  // the previous token's reads of s_k, s_u are done

        if (t < D) {
            const float kv = ld(k + t), qv = ld(q + t);
            s_k[t] = kv;
            s_q[t] = qv;
            s_alpha[t] = __expf(fmaxf(ld(g + t), a.lower_bound));
            const float kq = wave_sum(kv * qv);
            if (lane == 0) s_kq[wave] = kq;
        }
        __syncthreads();

        // Retention on rows, then the two column sums over this thread's rows.
        f32x4 pk[kQ], pq[kQ];
#pragma unroll
        for (int j = 0; j < kQ; ++j) pk[j] = pq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int r = rg + kRowGroups * i;
            const float al = s_alpha[r], kr = s_k[r], qr = s_q[r];
#pragma unroll
            for (int j = 0; j < kQ; ++j) {
                s[i][j] *= al;
                pk[j] += s[i][j] * kr;
                pq[j] += s[i][j] * qr;
            }
        }
        // lanes that hold the same columns for other row groups of the wavefront
#pragma unroll
        for (int m = M::kLanesPerRow; m < 64; m *= 2)
#pragma unroll
            for (int j = 0; j < kQ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk[j][e] += __shfl_xor(pk[j][e], m, 64);
                    pq[j][e] += __shfl_xor(pq[j][e], m, 64);
                }
        if (lane < M::kLanesPerRow) {
#pragma unroll
            for (int j = 0; j < kQ; ++j) {
                *reinterpret_cast<f32x4*>(&s_part[wave][0][c0 + 4 * j]) = pk[j];
                *reinterpret_cast<f32x4*>(&s_part[wave][1][c0 + 4 * j]) = pq[j];
            }
        }
        __syncthreads();

        if (t < D) {
            const int j = t;
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                sk += s_part[w][0][j];
                sq += s_part[w][1][j];
            }
            const float beta = ld(static_cast<const TIN*>(a.beta) + row);
            const float vj = ld(static_cast<const TIN*>(a.v) + row * D + j);
            const float u = beta * (vj - sk);
            s_u[j] = u;
            const float kq = s_kq[0] + s_kq[1];
            st(static_cast<TOUT*>(a.o) + row * D + j, a.scale * (sq + u * kq));
        }
        __syncthreads();

        f32x4 u4[kQ];
#pragma unroll
        for (int j = 0; j < kQ; ++j) u4[j] = *reinterpret_cast<const f32x4*>(&s_u[c0 + 4 * j]);
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const float kr = s_k[rg + kRowGroups * i];
#pragma unroll
            for (int j = 0; j < kQ; ++j) s[i][j] += kr * u4[j];
        }
        // the state after this token: every token's to token_states, else
        // only the last one, in place
        TS* dst = a.token_states ? static_cast<TS*>(a.token_states) + row * D * D : (tk + 1 == a.Tq ? Sp : nullptr);
        if (dst) {
#pragma unroll
            for (int i = 0; i < kRows; ++i) st_state(dst + (size_t)(rg + kRowGroups * i) * D + c0, s[i]);
        }
    }
}

// state[b, h] <- token_states[b, accepted[b] - 1, h]; 256 threads copy one
// state (64 or 32 KiB) with 16-byte accesses
template <int ES>
__global__ __launch_bounds__(256) void commit_kernel(const uint8_t* ts, const int32_t* accepted, uint8_t* state,
                                                      int Tq, int H)
{
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int acc = accepted[b];
    if (acc < 1 || acc > Tq) return;  // nothing accepted (or out of range): the state stays
    constexpr size_t kBytes = (size_t)D * D * ES;
    const f32x4* src = reinterpret_cast<const f32x4*>(ts + (((size_t)b * Tq + acc - 1) * H + h) * kBytes);
    f32x4* dst = reinterpret_cast<f32x4*>(state + (size_t)bh * kBytes);
#pragma unroll
    for (int i = 0; i < (int)(kBytes / 16 / 256); ++i) dst[threadIdx.x + 256 * i] = src[threadIdx.x + 256 * i];
}

// element-wise float32 <-> bfloat16 (or a copy), four elements per thread
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void convert_kernel(const TA* src, TB* dst, int64_t n)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        st4(dst + i, ld4(src + i));
    } else {
        for (int64_t j = i; j < n; ++j) st(dst + j, ld(src + j));
    }
}

template <typename TIN, typename TS>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)((int64_t)a.B * a.H)), block(Map<TS>::kThreads);
    if (a.out_dtype == F32)
        hipLaunchKernelGGL((decode_kernel<TIN, float, TS>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<TIN, bf16_t, TS>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s)
{
    if (a.state_dtype == F32) return a.in_dtype == F32 ? launch_t<float, float>(a, s) : launch_t<bf16_t, float>(a, s);
    return a.in_dtype == F32 ? launch_t<float, bf16_t>(a, s) : launch_t<bf16_t, bf16_t>(a, s);
}

hipError_t launch_decode_commit(const void* token_states, const int32_t* accepted, void* state, int B, int Tq, int H,
                                DType state_dtype, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)B * H)), block(256);
    const uint8_t* ts = static_cast<const uint8_t*>(token_states);
    uint8_t* st = static_cast<uint8_t*>(state);
    if (state_dtype == F32)
        hipLaunchKernelGGL(commit_kernel<4>, grid, block, 0, s, ts, accepted, st, Tq, H);
    else
        hipLaunchKernelGGL(commit_kernel<2>, grid, block, 0, s, ts, accepted, st, Tq, H);
    return hipGetLastError();
}

hipError_t launch_convert(const void* src, DType src_dtype, void* dst, DType dst_dtype, int64_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 1023) / 1024)), block(256);
    if (src_dtype == F32 && dst_dtype == BF16)
        hipLaunchKernelGGL((convert_kernel<float, bf16_t>), grid, block, 0, s, static_cast<const float*>(src),
                           static_cast<bf16_t*>(dst), n);
    else if (src_dtype == BF16 && dst_dtype == F32)
        hipLaunchKernelGGL((convert_kernel<bf16_t, float>), grid, block, 0, s, static_cast<const bf16_t*>(src),
                           static_cast<float*>(dst), n);
    else if (src_dtype == F32)
        hipLaunchKernelGGL((convert_kernel<float, float>), grid, block, 0, s, static_cast<const float*>(src),
                           static_cast<float*>(dst), n);
    else
        hipLaunchKernelGGL((convert_kernel<bf16_t, bf16_t>), grid, block, 0, s, static_cast<const bf16_t*>(src),
                           static_cast<bf16_t*>(dst), n);
    return hipGetLastError();
}

}  // namespace kda
