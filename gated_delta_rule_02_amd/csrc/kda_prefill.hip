// kda_prefill.hip -- single-pass chunked KDA prefill over packed sequences.
//
// The chunk form, its overflow-safe factorisation and the chunk-local phases
// P0 .. P2b are in kda_chunk.h. Here one workgroup of 8 wavefronts owns one
// (sequence, head) for the whole sequence: wavefront w owns value columns
// 16w .. 16w + 15 and keeps its 128 x 16 float32 slice of the state in
// registers (value columns of the state evolve independently). After P2b,
//   P3  every wavefront runs its own value-side chain (X, block forward
//       substitution, O, state update) on MFMA with no further barrier.
// Global accesses go through buffer descriptors whose byte range ends at the
// chunk's last valid row: loads past it return zero and stores are dropped,
// so ragged chunks need no masks or branches. The next chunk's inputs are
// loaded into registers while a chunk computes. This path needs no workspace;
// the two-pass path in kda_prefill_split.hip spreads the chunk-local work over
// the whole GPU when a workspace is given.
#include "kda_chunk.h"

namespace kda {
namespace {

template <bool F32P, typename TIN, typename TOUT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a)
{
    using O = Ops<F32P>;
    using F4 = typename O::F4;
    using F8 = typename O::F8;
    using SM = Smem<F32P>;
    using IN = Io<TIN>;
    constexpr int C = SM::C;
    constexpr int NB = SM::NB;
    constexpr int ES = sizeof(TIN);

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m16 = lane & 15;
    const int q4 = lane >> 4;

    const int bid = blockIdx.x;
    const int h = bid % a.H;
    const int n = bid / a.H;
    const int jcol = wave * 16 + m16;  // this lane's value column

    int64_t seq_s, seq_e;
    if (a.cu_seqlens) {
        seq_s = a.cu_seqlens[n];
        seq_e = a.cu_seqlens[n + 1];
    } else {
        seq_s = (int64_t)n * a.seq_len;
        seq_e = seq_s + a.seq_len;
    }

    // state slice: S[t][i] = S[16t + 4q + i][jcol]
    f32x4 S[8];
    const size_t sbase = ((size_t)n * a.H + h) * D * D;
    if (a.s0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] = a.s0[sbase + (size_t)(16 * t + 4 * q4 + i) * D + jcol];
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int ts = a.H * D;  // token stride in elements
    const TIN* vg = static_cast<const TIN*>(a.v);
    TOUT* og = static_cast<TOUT*>(a.o);

    Front<F32P, TIN> fr(sm, a, h);
    uint32_t rv[NB][4];  // v[16R + 4q + i][jcol] (raw bits)
    auto load_v = [&](int64_t c_s, int nt) {  // consumed in P3
        const rsrc_t rv_ = make_rsrc(vg + c_s * ts, (int64_t)nt * ts * ES);
        const int voff = (4 * q4 * ts + h * D + jcol) * ES;
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr)
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[Rr][i] = IN::ld_one(rv_, voff, (16 * Rr + i) * ts * ES);
    };
    if (seq_s < seq_e) {
        fr.load(seq_s, (int)min<int64_t>(C, seq_e - seq_s));
        load_v(seq_s, (int)min<int64_t>(C, seq_e - seq_s));
    }

    int64_t snap_next = a.snap_interval;  // tokens of the sequence at the next snapshot
    int64_t snap_j = 0;                   // its index
    for (int64_t cs = seq_s; cs < seq_e; cs += C) {
        const int ntok = (int)min<int64_t>(C, seq_e - cs);

        // ---------------- P0: half-block sums of the log-retention (base 2)
        fr.p0();
        __syncthreads();

        // ---------------- P1: decay factors and key-side operands
        fr.p1();
        // the next chunk's key-side inputs stream in while this chunk computes
        if (cs + C < seq_e) fr.load(cs + C, (int)min<int64_t>(C, seq_e - cs - C));
        __syncthreads();

        // ---------------- P2: blocks of A and P, diagonal inverses
        fr.p2();
        __syncthreads();

        // ---------------- P2b: k o 2^b, q o 2^b over the dead float32 region
        fr.p2b();
        __syncthreads();

        // ---------------- P3: value side, one 16-column tile per wavefront
        F4 sb[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) sb[t] = O::cvt(S[t]);
        f32x4 X[NB], O1[NB];
        F4 UB[NB];
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr) {
            f32x4 accX = {0.f, 0.f, 0.f, 0.f}, accO = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = 32 * s + 4 * q4;
                const F8 b = O::cat2(sb[2 * s], sb[2 * s + 1]);
                accX = O::mma32(O::cat2(O::lds(&sm.key.h.Kt[16 * Rr + m16][c]), O::lds(&sm.key.h.Kt[16 * Rr + m16][c + 16])), b, accX);
                accO = O::mma32(O::cat2(O::lds(&sm.key.h.Qt[16 * Rr + m16][c]), O::lds(&sm.key.h.Qt[16 * Rr + m16][c + 16])), b, accO);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * Rr + 4 * q4 + i;  // rows past the chunk: v = beta = 0
                X[Rr][i] = sm.beta[r] * (IN::one(rv[Rr][i]) - accX[i]);
            }
            O1[Rr] = accO;
            __builtin_amdgcn_sched_barrier(0);  // bound the scheduler's look-ahead (register pressure)
        }
        // block forward substitution: U_R = T_RR (X_R - sum_{I<R} A_RI U_I)
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr) {
            f32x4 Y = X[Rr];
#pragma unroll
            for (int I = 0; I + 1 < Rr; I += 2)
                Y = O::mma32(O::cat2(O::lds(&sm.An[pair_id(Rr, I)][m16][4 * q4]), O::lds(&sm.An[pair_id(Rr, I + 1)][m16][4 * q4])),
                             O::cat2(UB[I], UB[I + 1]), Y);
            if (Rr & 1) Y = O::mma16(O::lds(&sm.An[pair_id(Rr, Rr - 1)][m16][4 * q4]), UB[Rr - 1], Y);
            const f32x4 U = O::mma16(O::lds(&sm.Tb[Rr][m16][4 * q4]), O::cvt(Y), f32x4{0.f, 0.f, 0.f, 0.f});
            UB[Rr] = O::cvt(U);
        }
        // outputs O_R = scale (O1_R + sum_{I<=R} P_RI U_I); rows past the chunk are dropped
        const rsrc_t ro_ = make_rsrc(og + cs * ts, (int64_t)ntok * ts * (int64_t)sizeof(TOUT));
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr) {
            f32x4 acc = O1[Rr];
#pragma unroll
            for (int I = 0; I + 1 <= Rr; I += 2)
                acc = O::mma32(O::cat2(O::lds(&sm.Pb[tri_id(Rr, I)][m16][4 * q4]), O::lds(&sm.Pb[tri_id(Rr, I + 1)][m16][4 * q4])),
                               O::cat2(UB[I], UB[I + 1]), acc);
            if (!(Rr & 1)) acc = O::mma16(O::lds(&sm.Pb[tri_id(Rr, Rr)][m16][4 * q4]), UB[Rr], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Io<TOUT>::st(ro_, (4 * q4 * ts + h * D + jcol) * (int)sizeof(TOUT), (16 * Rr + i) * ts * (int)sizeof(TOUT),
                             a.scale * acc[i]);
        }
        // state: S <- Diag(2^b_C) S + Kbar^T U
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            f32x4 acc = S[t] * ld4f(&sm.bC[16 * t + 4 * q4]);
#pragma unroll
            for (int Rr = 0; Rr < NB; Rr += 2)
                acc = O::mma32(O::cat2(O::lds(&sm.KbT[16 * t + m16][16 * Rr + 4 * q4]), O::lds(&sm.KbT[16 * t + m16][16 * Rr + 16 + 4 * q4])),
                               O::cat2(UB[Rr], UB[Rr + 1]), acc);
            S[t] = acc;
        }
        // state snapshot when a whole chunk ends on a multiple of the interval
        if (a.snap && cs + C - seq_s == snap_next && cs + C <= seq_e) {
            store_state_slice(a.snap + (((size_t)n * a.snap_slots + snap_j) * a.H + h) * D * D, S, q4, jcol);
            snap_next += a.snap_interval;
            ++snap_j;
        }
        if (cs + C < seq_e) load_v(cs + C, (int)min<int64_t>(C, seq_e - cs - C));
        __syncthreads();
    }

    if (a.sT) {
        // the empty asm keeps the compiler from computing these addresses before
        // the chunk loop and holding them in registers across it
        int off = 4 * q4 * D + jcol;
        asm volatile("" : "+v"(off));
        float* sT = a.sT + sbase + off;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * t + i) * D] = S[t][i];
    }
}

template <bool F32P, typename TIN>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.H)), block(kThreads);
    if (a.out_dtype == F32)
        hipLaunchKernelGGL((prefill_kernel<F32P, TIN, float>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((prefill_kernel<F32P, TIN, bf16_t>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s)
{
    return a.in_dtype == F32 ? launch_t<true, float>(a, s) : launch_t<false, bf16_t>(a, s);
}

}  // namespace kda
