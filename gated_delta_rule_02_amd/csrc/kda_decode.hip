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
// Workgroup = 1024 threads = one (sequence, head). Thread t owns the 4 columns
// 4*(t%32) .. +3 of the 4 rows r = t/32 + 32*i (i = 0..3): a wavefront's 64
// lanes cover two whole rows, i.e. 1 KiB of contiguous state per load.
// Measured on the 1 GiB decode workload: 256 threads x 16 rows 410 us,
// 512 x 8 410 us, 1024 x 4 386 us (the in-place stream of the state is the
// whole cost; the wider workgroup keeps more of it in flight).
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
constexpr int kThreads = KDA_DECODE_THREADS;   // per (sequence, head)
constexpr int kWaves = kThreads / 64;
constexpr int kRowGroups = kThreads / 32;      // 32 lanes cover one 128-float row
constexpr int kRowsPerThread = D / kRowGroups;

template <typename TIN, typename TOUT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a)
{
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
    // owns columns 4 (t % 32) .. +3 of the rows t / 32 + kRowGroups i.
    const int cg = t & 31;
    const int rg = t >> 5;
    float* Sp = a.state + (size_t)bh * D * D;
    f32x4 s[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
        s[i] = KDA_NT_LOAD(reinterpret_cast<const f32x4*>(Sp + (size_t)(rg + kRowGroups * i) * D + 4 * cg));

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
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) {
            const int r = rg + kRowGroups * i;
            s[i] *= s_alpha[r];
            pk += s[i] * s_k[r];
            pq += s[i] * s_q[r];
        }
        // lanes l and l^32 hold the same columns for adjacent row groups
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pk[j] += __shfl_xor(pk[j], 32, 64);
            pq[j] += __shfl_xor(pq[j], 32, 64);
        }
        if (lane < 32) {
            *reinterpret_cast<f32x4*>(&s_part[wave][0][4 * cg]) = pk;
            *reinterpret_cast<f32x4*>(&s_part[wave][1][4 * cg]) = pq;
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

        const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cg]);
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) s[i] += s_k[rg + kRowGroups * i] * u4;
        // the state after this token: every token's to token_states, else
        // only the last one, in place
        float* dst = a.token_states ? a.token_states + row * D * D : (tk + 1 == a.Tq ? Sp : nullptr);
        if (dst) {
#pragma unroll
            for (int i = 0; i < kRowsPerThread; ++i)
                KDA_NT_STORE(s[i], reinterpret_cast<f32x4*>(dst + (size_t)(rg + kRowGroups * i) * D + 4 * cg));
        }
    }
}

// state[b, h] <- token_states[b, accepted[b] - 1, h]; 256 threads copy one
// 64 KiB state with 16-byte accesses
__global__ __launch_bounds__(256) void commit_kernel(const float* ts, const int32_t* accepted, float* state, int Tq,
                                                      int H)
{
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int acc = accepted[b];
    if (acc < 1 || acc > Tq) return;  // nothing accepted (or out of range): the state stays
    const f32x4* src = reinterpret_cast<const f32x4*>(ts + (((size_t)b * Tq + acc - 1) * H + h) * D * D);
    f32x4* dst = reinterpret_cast<f32x4*>(state + (size_t)bh * D * D);
#pragma unroll
    for (int i = 0; i < D * D / 4 / 256; ++i) dst[threadIdx.x + 256 * i] = src[threadIdx.x + 256 * i];
}

template <typename TIN>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)((int64_t)a.B * a.H)), block(kThreads);
    if (a.out_dtype == F32)
        hipLaunchKernelGGL((decode_kernel<TIN, float>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<TIN, bf16_t>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s)
{
    return a.in_dtype == F32 ? launch_t<float>(a, s) : launch_t<bf16_t>(a, s);
}

hipError_t launch_decode_commit(const float* token_states, const int32_t* accepted, float* state, int B, int Tq,
                                int H, hipStream_t s)
{
    hipLaunchKernelGGL(commit_kernel, dim3((unsigned)((int64_t)B * H)), dim3(256), 0, s, token_states, accepted,
                       state, Tq, H);
    return hipGetLastError();
}

}  // namespace kda
