// kda_chunk.h -- the chunk-local phases of the KDA prefill on gfx950, shared
// by the single-pass kernel (kda_prefill.hip) and the two-pass kernels
// (kda_prefill_split.hip).
//
// Computes, per (sequence, head), the recurrence of "Ling-3.1-flash: Grouped
// Routing and Two Different MLA Caches" (flozi.net), section "KDA replaces a
// token list with a recurrent matrix" (retention per key channel, delta-rule
// write, read after the write), reorganised exactly over chunks of C tokens.
//
// The chunk form. For a chunk with start state S0 (dk x dv) and tokens
// r = 0..C-1, let b_r = sum_{j<=r} g_j (per key channel, here in base 2). Then
//   A[r,i] = beta_r sum_c k_rc k_ic 2^(b_rc - b_ic)   (i < r)
//   U      = (I + A)^-1 X,    X = diag(beta) (V - (K o 2^B) S0)
//   P[r,i] = sum_c q_rc k_ic 2^(b_rc - b_ic)           (i <= r)
//   O      = scale ((Q o 2^B) S0 + P U)
//   S_C    = Diag(2^b_C) S0 + (K o 2^(b_C - B))^T U
// U are the corrected writes u_r = beta_r (v_r - S'_r^T k_r) of all tokens of
// the chunk; the triangular solve replaces the token-serial dependency.
//
// Overflow-safe factorisation. The chunk is cut into NB = C/16 blocks of 16
// tokens. With rho_R the cumulative log-retention before block R, l_r the
// inclusive prefix sum inside r's block, s_i the sum over the tokens after i in
// i's block, and G_R the block total:
//   b_r - b_i = l_r + (rho_R - rho_{I+1}) + s_i   (i in block I < R: all <= 0)
//   b_r - b_i = l_r + s_i - G_R                   (i, r in the same block R)
// Every factor 2^x of a block product then spans the clamped log-retentions of
// at most one block (16 tokens), so |x| <= 16 |lower_bound| log2(e): 115.4 at
// the -5 floor of the safe forget gate (flozi.net section above), and 124.7 at
// -5.4, the lowest floor the library accepts, which keeps every factor a
// normal float32 (neither infinite nor subnormal).
//
// Work split. A workgroup of 8 wavefronts handles one chunk at a time:
//   P0  each producer thread (2 key channels, a row group of a 16-token
//       block) sums its log-retentions; the partial sums go through LDS.
//   P1  it forms the decay factors by running products of alpha = 2^g and
//       writes the key-side operands k o 2^l, q o 2^l, k o 2^s (float32) and
//       the transposed K-bar (operand type); it keeps k o 2^b and q o 2^b
//       (operand type) in registers.
//   P2  wavefronts 0..NB-1 compute the diagonal blocks of A and P and the
//       diagonal inverses; the others compute the off-diagonal blocks.
//   P2b the float32 region is dead: k o 2^b and q o 2^b are written over it.
// The value side that follows P2b differs between the two kernels.
//
// Precision (bfloat16 inputs): the key-side operands are staged in LDS as
// float32 and rounded once per use. Off-diagonal blocks and the whole value
// side run float16 MFMA (their operands are bounded by 1 or by the state and
// value magnitudes, so float16's range suffices and its 11-bit significand
// keeps the error well inside the bound); A's diagonal blocks use bfloat16
// (their right operand reaches 2^116); P's diagonal blocks use a hi+lo
// bfloat16 split (3 MFMAs) because they dominate the output error otherwise.
// Accumulation, the state and all exponents are float32. Float32 inputs run a
// float32-MFMA variant with 32-token chunks.
#pragma once
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {


constexpr int D = 128;  // dk = dv
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
template <typename T> struct Io;
// Loads take a cache policy: kStream (the non-temporal hint) for data that is
// read or written exactly once, so that it does not displace data still to be
// reused from the caches. The two-pass prefill streams its inputs in and its
// outputs out when a window's workspace fits the last-level cache, which then
// keeps that workspace for the state pass: with the caches flushed before each
// call (512 MiB written) the 4096-token call ran 0.278 ms with ordinary
// accesses and 0.212 ms with these hints (0.204 and 0.206 ms without the
// flush). When the workspace is far larger than the cache the hints only cost
// (the packed varlen workload: 7.12 ms against 7.35 ms).
constexpr int kStream = 2;
template <> struct Io<bf16_t> {
    using pair_t = uint32_t;
    template <int Pol = 0>
    __device__ static pair_t ld_pair(rsrc_t r, int off, int soff) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, Pol); }
    __device__ static f32x2 unpack(pair_t u) { return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)}; }
    template <int Pol = 0>
    __device__ static uint32_t ld_one(rsrc_t r, int off, int soff) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, Pol); }
    __device__ static float one(uint32_t u) { return __uint_as_float(u << 16); }
    __device__ static void st(rsrc_t r, int off, int soff, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), r, off, soff, 0);
    }
};
template <> struct Io<float> {
    using pair_t = uint2;
    template <int Pol = 0>
    __device__ static pair_t ld_pair(rsrc_t r, int off, int soff)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, Pol);
        return make_uint2(v[0], v[1]);
    }
    __device__ static f32x2 unpack(pair_t u) { return f32x2{__uint_as_float(u.x), __uint_as_float(u.y)}; }
    template <int Pol = 0>
    __device__ static uint32_t ld_one(rsrc_t r, int off, int soff) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, Pol); }
    __device__ static float one(uint32_t u) { return __uint_as_float(u); }
    __device__ static void st(rsrc_t r, int off, int soff, float v)
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, soff, 0);
    }
};

// ---------------------------------------------------------------- MFMA ops
// Operand layout of the 16 x 16 MFMAs used here. A K16 slab: lane
// (m = lane % 16, q = lane / 16) holds A[m][4q..4q+3] and B[4q..4q+3][n = m];
// the 16 x 16 result holds C[4q+i][n] in element i. A K32 step concatenates
// two K16 slabs per lane (elements 0-3 from the first, 4-7 from the second);
// A and B use the same assignment, so the product sums every k exactly once.
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// A wavefront's 128 x 16 slice of a float32 128 x 128 state, held as
// S[t][i] = S[16t + 4q + i][jcol], written to the state at `dst` (row major)
__device__ __forceinline__ void store_state_slice(float* dst, const f32x4 (&S)[8], int q4, int jcol)
{
    float* p = dst + 4 * q4 * D + jcol;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[(16 * t + i) * D] = S[t][i];
}

__device__ __forceinline__ h4 to_h4(f32x4 x)
{
    return h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ b4 to_b4(f32x4 x)
{
    return b4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
__device__ __forceinline__ f32x4 from_b4(b4 x)
{
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ h8 cat(h4 a, h4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ b8 cat(b4 a, b4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ __forceinline__ f32x4 mma_f32_k16(f32x4 a, f32x4 b, f32x4 c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

template <bool F32P> struct Ops;

// bfloat16 inputs: float16 operands (bfloat16 for the diagonal blocks)
template <> struct Ops<false> {
    using OT = _Float16;
    using F4 = h4;
    using F8 = h8;
    static constexpr int C = 64;
    static constexpr int PAD = 8;
    __device__ static F4 cvt(f32x4 x) { return to_h4(x); }
    __device__ static F8 cat2(F4 a, F4 b) { return cat(a, b); }
    __device__ static F4 lds(const OT* p) { return *reinterpret_cast<const h4*>(p); }
    // Only the 16x16x32 instruction form is used: dependent chains that mixed
    // the 16x16x16 and 16x16x32 forms returned stale accumulator elements on
    // gfx950, so a K16 step is the K32 instruction with a zero second half.
    __device__ static f32x4 mma16(F4 a, F4 b, f32x4 c)
    {
        const F4 z = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(cat(a, z), cat(b, z), c, 0, 0, 0);
    }
    __device__ static f32x4 mma32(F8 a, F8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
    // A's diagonal blocks: one bfloat16 product (operands up to 2^116)
    __device__ static f32x4 diagA(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat(to_b4(a0), to_b4(a1)), cat(to_b4(b0), to_b4(b1)), c, 0, 0, 0);
    }
    // P's diagonal blocks: hi + lo bfloat16 split of both operands (3 products)
    __device__ static f32x4 diagP(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 c)
    {
        const b4 ah0 = to_b4(a0), ah1 = to_b4(a1), bh0 = to_b4(b0), bh1 = to_b4(b1);
        const b8 ah = cat(ah0, ah1), bh = cat(bh0, bh1);
        const b8 al = cat(to_b4(a0 - from_b4(ah0)), to_b4(a1 - from_b4(ah1)));
        const b8 bl = cat(to_b4(b0 - from_b4(bh0)), to_b4(b1 - from_b4(bh1)));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
        return c;
    }
    // two operand-type values of channels c, c+1 packed for one LDS store
    using P2 = h2;
    __device__ static P2 pack2(float x, float y) { return h2{(_Float16)x, (_Float16)y}; }
    // N consecutive tokens of one channel for the transposed K-bar
    template <int N>
    __device__ static void store_n(OT* p, const float* v)
    {
        static_assert(N == 4 || N == 8, "4 or 8 tokens");
        if constexpr (N == 8)
            *reinterpret_cast<h8*>(p) = h8{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3],
                                           (_Float16)v[4], (_Float16)v[5], (_Float16)v[6], (_Float16)v[7]};
        else
            *reinterpret_cast<h4*>(p) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    }
};

// float32 inputs: float32 MFMA throughout
struct F32x8 {
    f32x4 a, b;
};
template <> struct Ops<true> {
    using OT = float;
    using F4 = f32x4;
    using F8 = F32x8;
    static constexpr int C = 32;
    static constexpr int PAD = 4;
    __device__ static F4 cvt(f32x4 x) { return x; }
    __device__ static F8 cat2(F4 a, F4 b) { return F8{a, b}; }
    __device__ static F4 lds(const OT* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ static f32x4 mma16(F4 a, F4 b, f32x4 c) { return mma_f32_k16(a, b, c); }
    __device__ static f32x4 mma32(F8 a, F8 b, f32x4 c) { return mma_f32_k16(a.b, b.b, mma_f32_k16(a.a, b.a, c)); }
    __device__ static f32x4 diagA(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 c)
    {
        return mma_f32_k16(a1, b1, mma_f32_k16(a0, b0, c));
    }
    __device__ static f32x4 diagP(f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1, f32x4 c)
    {
        return mma_f32_k16(a1, b1, mma_f32_k16(a0, b0, c));
    }
    using P2 = f32x2;
    __device__ static P2 pack2(float x, float y) { return f32x2{x, y}; }
    template <int N>
    __device__ static void store_n(OT* p, const float* v)
    {
        static_assert(N == 4 || N == 8, "4 or 8 tokens");
        *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
        if constexpr (N == 8) *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
};

// Row stride of the 16 x 16 blocks: four elements of padding, so that the
// A-layout reads (lane m reads four or eight bytes of row m) of a wavefront's
// 16 rows fall in distinct LDS banks (with a stride of 16 every fourth row
// shares a bank, a four-way conflict).
constexpr int BLD = 20;

// index of the off-diagonal block pair (R, I), I < R
__host__ __device__ constexpr int pair_id(int R, int I) { return R * (R - 1) / 2 + I; }
// index of the lower-triangle block (R, I), I <= R
__host__ __device__ constexpr int tri_id(int R, int I) { return R * (R + 1) / 2 + I; }

// NQ: producer row groups per 16-token block (16 / NQ tokens per producer thread)
template <bool F32P, int NQ = 2>
struct __attribute__((aligned(16))) Smem {
    using OT = typename Ops<F32P>::OT;
    static constexpr int C = Ops<F32P>::C;
    static constexpr int NB = C / 16;
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr int LDK = D + 4;               // row stride of the float32 [C][128] arrays
    static constexpr int LDH = D + Ops<F32P>::PAD;  // row stride of the operand-type [C][128] arrays
    static constexpr int LDT = C + Ops<F32P>::PAD;  // row stride of [128][C]
    OT Nd[NB][16][BLD];                     // -A diagonal blocks (strictly lower, beta-scaled)
    OT Tb[NB][16][BLD];                     // (I + A_RR)^-1
    OT An[NPAIR > 0 ? NPAIR : 1][16][BLD];  // -A off-diagonal blocks (beta-scaled)
    OT Pb[NB * (NB + 1) / 2][16][BLD];      // P lower-triangle blocks
    float Fd[NB][D];                        // 2^-G_R
    float Fo[NPAIR > 0 ? NPAIR : 1][D];     // 2^(rho_R - rho_{I+1})
    float Gp[NB][NQ][D];                    // row-group sums of the log-retention (base 2)
    float bC[D];                            // 2^b_C
    float beta[C];
    OT KbT[D][LDT];                         // (k o 2^(b_C - b))^T   (state update)
    // P1 -> P2: key-side operands in float32. Their factors span 2^-116 .. 1
    // and the diagonal blocks rescale them by up to 2^116, beyond float16's
    // range, so each use rounds once to the MFMA operand type.
    // P2b -> P3: the same bytes then hold k o 2^b and q o 2^b (operand type).
    // The small tables come first so that their LDS offsets fit the
    // instructions' immediate offset field.
    union Key {
        struct {
            float KL[C][LDK];  // k o 2^l   (left operand of A)
            float QL[C][LDK];  // q o 2^l   (left operand of P)
            float KS[C][LDK];  // k o 2^s   (right operand of A and P)
        } f;
        struct {
            OT Kt[C][LDH];     // k o 2^b   (X = diag(beta)(V - Kt S))
            OT Qt[C][LDH];     // q o 2^b   (O = Qt S + P U)
        } h;
        // two-pass form: the right-hand sides of the products with
        // T = (I + A)^-1, transposed ([channel][token], so that a lane reads
        // four consecutive tokens of its channel at once), and Q~
        struct {
            OT XWt[D][LDT];    // (-diag(beta) (K o 2^B))^T
            OT XUt[D][LDT];    // (diag(beta) V)^T
            OT Qt[C][LDH];     // q o 2^b
        } x;
    } key;
};


// ---------------------------------------------------------------- P0 .. P2b
// The chunk-local phases. Producer threads (wavefronts 0 .. NQ NB - 1) own
// channels c0, c0 + 1 of the RP = 16 / NQ tokens rbase .. rbase + RP - 1 (row
// group hh of block R); the next chunk's k, q, g of those tokens and beta
// stream into registers while the current chunk computes. The caller
// separates the phases with barriers.
// NoQ: no query side (the segment maps of the sequence-parallel prefill form
// no output): q is not loaded and neither P nor q o 2^b is formed.
// Gate: the gate prologue runs here (PrefillArgs::gate_f): the g and beta
// loads read the projection rows f and b, and P0 forms g and beta from them,
// rounded to bfloat16 exactly as the gate prologue stores them, so the results
// equal those of the prologue followed by the prefill.
// Lean: the two-pass intra pass. The kernel holds no state in registers
// here, so P2 can afford more live registers: the diagonal-block inverses by
// repeated squaring instead of the Horner form (fewer dependent products) and
// the off-diagonal pairs split evenly over the SIMDs. The producers also load
// v and, in P2b, stage the right-hand sides -diag(beta)(K o 2^B) and
// diag(beta) V of the products with T, transposed and rounded once.
template <bool F32P, typename TIN, int NQ = 2, bool Lean = false, int LoadPol = 0, bool NoQ = false,
          bool Gate = false>
struct Front {
    using O = Ops<F32P>;
    using OT = typename O::OT;
    using F4 = typename O::F4;
    using F8 = typename O::F8;
    using SM = Smem<F32P, NQ>;
    using IN = Io<TIN>;
    using PT = typename IN::pair_t;
    static constexpr int C = SM::C;
    static constexpr int NB = SM::NB;
    static constexpr int RP = 16 / NQ;  // tokens per producer thread
    static constexpr int ES = sizeof(TIN);

    SM& sm;
    const int tid, wave, lane, m16, q4;
    const bool prod;
    const int R, hh, c0, rbase;
    const int h, H, ts;
    const float lbl;
    const TIN *qg, *kg, *gg, *bg;
    const int64_t gts, bts;   // row strides (elements) of the g and beta sources
    const float lb, rate;     // Gate: lower bound, exp(A_log[h])
    int ntl = 0;              // Gate: tokens of the loaded chunk (rows past it get g = 0)

    PT rk[RP], rq[RP], rg[RP];  // k, q, g of this producer's tokens
    PT rvv[Lean ? RP : 1];      // v of this producer's tokens (Lean)
    uint32_t rb = 0;            // beta[tid] (threads < C)
    f32x2 g2[RP];               // clamped base-2 log-retention
    // k o 2^b (or, Lean, -beta k o 2^b) and q o 2^b of this producer's tokens
    typename O::P2 kt2[RP], qt2[RP];
    typename O::P2 xu2[Lean ? RP : 1];  // Lean: beta v of this producer's tokens

    // the wavefront index is read through readfirstlane so that the compiler
    // knows every quantity derived from it is wave-uniform (scalar offsets)
    __device__ __forceinline__ Front(SM& s, const PrefillArgs& a, int head)
        : sm(s), tid(threadIdx.x), wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)), lane(threadIdx.x & 63),
          m16(threadIdx.x & 15), q4((threadIdx.x & 63) >> 4), prod(wave < NQ * NB), R(wave % NB), hh(wave / NB),
          c0(2 * (threadIdx.x & 63)), rbase(16 * (wave % NB) + RP * (wave / NB)), h(head), H(a.H), ts(a.H * D),
          lbl(a.lower_bound * kLog2e), qg(static_cast<const TIN*>(a.q)), kg(static_cast<const TIN*>(a.k)),
          gg(static_cast<const TIN*>(Gate ? a.gate_f : a.g)), bg(static_cast<const TIN*>(Gate ? a.gate_b : a.beta)),
          gts(Gate ? a.gate_f_ld : (int64_t)a.H * D), bts(Gate ? a.gate_b_ld : a.H), lb(a.lower_bound),
          rate(Gate ? __expf(a.A_log[head]) : 0.0f)
    {
    }

    // k, q, g, beta of the nt tokens starting at c_s (rows past nt read as 0)
    // (and v when Lean). Parts (bit mask): 1 = g, k and beta, 2 = q, 4 = v,
    // so that a caller can spread the issue of the next chunk's loads over
    // several phases.
    template <int Parts = 7>
    __device__ __forceinline__ void load(int64_t c_s, int nt, const TIN* vg = nullptr)
    {
        const int64_t bytes = (int64_t)nt * ts * ES;
        constexpr int Pol = LoadPol;  // cache policy of the input loads
        if (prod) {
            const int voff = (c0 + h * D) * ES;  // per lane
            if constexpr (Parts & 1) {
                const rsrc_t rk_ = make_rsrc(kg + c_s * ts, bytes);
                const rsrc_t rg_ = make_rsrc(gg + c_s * gts, (int64_t)nt * gts * ES);
#pragma unroll
                for (int t = 0; t < RP; ++t) {
                    const int soff = (rbase + t) * ts * ES;  // wave-uniform row term
                    rg[t] = IN::template ld_pair<Pol>(rg_, voff, Gate ? (int)((rbase + t) * gts * ES) : soff);
                    rk[t] = IN::template ld_pair<Pol>(rk_, voff, soff);
                }
            }
            if constexpr ((Parts & 2) && !NoQ) {
                const rsrc_t rq_ = make_rsrc(qg + c_s * ts, bytes);
#pragma unroll
                for (int t = 0; t < RP; ++t) rq[t] = IN::template ld_pair<Pol>(rq_, voff, (rbase + t) * ts * ES);
            }
            if constexpr (Lean && (Parts & 4)) {
                const rsrc_t rv_ = make_rsrc(vg + c_s * ts, bytes);
#pragma unroll
                for (int t = 0; t < RP; ++t) rvv[t] = IN::template ld_pair<Pol>(rv_, voff, (rbase + t) * ts * ES);
            }
        }
        if constexpr (Parts & 1) {
            const rsrc_t rb_ = make_rsrc(bg + c_s * bts, (int64_t)nt * bts * ES);  // uniform: built outside the branch
            if (tid < C) rb = IN::template ld_one<Pol>(rb_, (int)((tid * bts + h) * ES), 0);
            if constexpr (Gate) ntl = nt;
        }
    }

    // P0: row-group sums of the log-retention (base 2), beta to LDS
    __device__ __forceinline__ void p0()
    {
        if (prod) {
            f32x2 G = {0.f, 0.f};
#pragma unroll
            for (int t = 0; t < RP; ++t) {
                f32x2 gv = IN::unpack(rg[t]);  // rows past the chunk read as 0
                if constexpr (Gate) {
                    // the gate prologue's g (stored as bfloat16); rows past the chunk 0
                    const bool live = rbase + t < ntl;
                    gv.x = live ? (float)(__bf16)fmaxf(-rate * softplus_hw(gv.x), lb) : 0.0f;
                    gv.y = live ? (float)(__bf16)fmaxf(-rate * softplus_hw(gv.y), lb) : 0.0f;
                }
                g2[t] = f32x2{fmaxf(gv.x * kLog2e, lbl), fmaxf(gv.y * kLog2e, lbl)};
                G += g2[t];
            }
            *reinterpret_cast<f32x2*>(&sm.Gp[R][hh][c0]) = G;
        }
        if (tid < C) {
            if constexpr (Gate)
                sm.beta[tid] = tid < ntl ? (float)(__bf16)sigmoidf_(IN::one(rb)) : 0.0f;
            else
                sm.beta[tid] = IN::one(rb);
        }
    }

    __device__ __forceinline__ f32x2 block_sum(int J) const
    {
        f32x2 g = {0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) g += *reinterpret_cast<const f32x2*>(&sm.Gp[J][qq][c0]);
        return g;
    }

    // P1: decay factors and key-side operands
    __device__ __forceinline__ void p1()
    {
        if (!prod) return;
        f32x2 rho_R = {0.f, 0.f}, bCv = {0.f, 0.f}, GR = {0.f, 0.f};
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            const f32x2 gJ = block_sum(J);
            if (J < R) rho_R += gJ;
            if (J == R) GR = gJ;
            bCv += gJ;
        }
        // sums of the row groups before / after this thread's inside the block
        f32x2 pre = {0.f, 0.f}, suf = {0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            const f32x2 x = *reinterpret_cast<const f32x2*>(&sm.Gp[R][qq][c0]);
            if (qq < hh) pre += x;
            if (qq > hh) suf += x;
        }
        if (hh == 0) {
            // factor tables for P2 and the value side (this thread's two channels)
            *reinterpret_cast<f32x2*>(&sm.Fd[R][c0]) = f32x2{exp2_fast(-GR.x), exp2_fast(-GR.y)};
            f32x2 rho_I1 = {0.f, 0.f};
#pragma unroll
            for (int I = 0; I < NB - 1; ++I) {
                rho_I1 += block_sum(I);
                if (I < R)  // pair (R, I): index R (R - 1) / 2 + I
                    *reinterpret_cast<f32x2*>(&sm.Fo[R * (R - 1) / 2 + I][c0]) =
                        f32x2{exp2_fast(rho_R.x - rho_I1.x), exp2_fast(rho_R.y - rho_I1.y)};
            }
            if (R == 0) *reinterpret_cast<f32x2*>(&sm.bC[c0]) = f32x2{exp2_fast(bCv.x), exp2_fast(bCv.y)};
        }
        const f32x2 DR = {exp2_fast(rho_R.x), exp2_fast(rho_R.y)};
        const f32x2 fb = {exp2_fast(bCv.x - rho_R.x - GR.x), exp2_fast(bCv.y - rho_R.y - GR.y)};

        // forward: e_l = prod_{j<=r} alpha_j over the block (starts after the earlier row groups)
        f32x2 al[RP];
#pragma unroll
        for (int t = 0; t < RP; ++t) al[t] = f32x2{exp2_fast(g2[t].x), exp2_fast(g2[t].y)};
        f32x2 el = {exp2_fast(pre.x), exp2_fast(pre.y)};
        float nb[RP];  // Lean: -beta of this producer's tokens (rows past the chunk: 0)
        if constexpr (Lean) {
#pragma unroll
            for (int t = 0; t < RP; t += 4) {
                const f32x4 b4v = ld4f(&sm.beta[rbase + t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) nb[t + i] = -b4v[i];
            }
        }
#pragma unroll
        for (int t = 0; t < RP; ++t) {
            el *= al[t];
            const f32x2 kv = IN::unpack(rk[t]), qv = NoQ ? f32x2{0.f, 0.f} : IN::unpack(rq[t]);
            const f32x2 klv = kv * el, qlv = qv * el;
            *reinterpret_cast<f32x2*>(&sm.key.f.KL[rbase + t][c0]) = klv;
            if constexpr (!NoQ) *reinterpret_cast<f32x2*>(&sm.key.f.QL[rbase + t][c0]) = qlv;
            if constexpr (Lean) {
                kt2[t] = O::pack2(klv.x * (DR.x * nb[t]), klv.y * (DR.y * nb[t]));
                const f32x2 vv = IN::unpack(rvv[t]);  // the next chunk's loads reuse rvv after P1
                xu2[t] = O::pack2(-nb[t] * vv.x, -nb[t] * vv.y);
            } else
                kt2[t] = O::pack2(klv.x * DR.x, klv.y * DR.y);
            qt2[t] = O::pack2(qlv.x * DR.x, qlv.y * DR.y);
        }
        // reverse: e_s = prod_{j>r} alpha_j over the block (starts before the later row groups)
        f32x2 es = {exp2_fast(suf.x), exp2_fast(suf.y)};
        float kb0[RP], kb1[RP];
#pragma unroll
        for (int t = RP - 1; t >= 0; --t) {
            const f32x2 ksv = IN::unpack(rk[t]) * es;
            *reinterpret_cast<f32x2*>(&sm.key.f.KS[rbase + t][c0]) = ksv;
            kb0[t] = ksv.x * fb.x;
            kb1[t] = ksv.y * fb.y;
            es *= al[t];
        }
        O::template store_n<RP>(&sm.KbT[c0][rbase], kb0);
        O::template store_n<RP>(&sm.KbT[c0 + 1][rbase], kb1);
    }

    // P2 pieces. Diagonal block Rd: A (bfloat16) and P (hi+lo split), the
    // beta-scaled strict lower part N and (I + N)^-1 by a Horner product.
    __device__ __forceinline__ void p2_diag(int Rd)
    {
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 32 * s + 4 * q4;
            const float* kl = &sm.key.f.KL[16 * Rd + m16][c];
            const float* ql = &sm.key.f.QL[16 * Rd + m16][c];
            const float* ks = &sm.key.f.KS[16 * Rd + m16][c];
            const f32x4 x0 = ld4f(ks) * ld4f(&sm.Fd[Rd][c]);
            const f32x4 x1 = ld4f(ks + 16) * ld4f(&sm.Fd[Rd][c + 16]);
            accA = O::diagA(ld4f(kl), ld4f(kl + 16), x0, x1, accA);
            if constexpr (!NoQ) accP = O::diagP(ld4f(ql), ld4f(ql + 16), x0, x1, accP);
            if constexpr (!Lean) __builtin_amdgcn_sched_barrier(0);  // one K step at a time (register pressure)
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q4 + i;  // row in block, column m16
            const float b = sm.beta[16 * Rd + row];
            sm.Nd[Rd][row][m16] = (OT)(row > m16 ? -accA[i] * b : 0.0f);
            if constexpr (!NoQ) sm.Pb[tri_id(Rd, Rd)][row][m16] = (OT)(row >= m16 ? accP[i] : 0.0f);
        }
        // wavefront-local: the inverse below reads what this wavefront wrote
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if constexpr (!Lean) {
            // (I + N)^-1 = sum_{j<16} (-N)^j  (N strictly lower, N^16 = 0), Horner form
            const F4 nA = O::lds(&sm.Nd[Rd][m16][4 * q4]);
            f32x4 eye;
#pragma unroll
            for (int i = 0; i < 4; ++i) eye[i] = (4 * q4 + i == m16) ? 1.0f : 0.0f;
            f32x4 Y = eye;
#pragma unroll
            for (int it = 0; it < 15; ++it) Y = O::mma16(nA, O::cvt(Y), eye);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.Tb[Rd][4 * q4 + i][m16] = (OT)Y[i];
            return;
        }
        // (I + A_RR)^-1 = sum_{j<16} M^j = (I + M)(I + M^2)(I + M^4)(I + M^8)
        // with M = -A_RR (strictly lower, M^16 = 0): three squarings and three
        // products instead of fifteen dependent Horner steps. A square needs
        // its operand in both layouts; the registers of X in the A layout are
        // those of X^T in the B layout, so X^2 and (X^2)^T = X^T X^T come from
        // the same two registers and fill both layouts of the next power.
        F4 aM = O::lds(&sm.Nd[Rd][m16][4 * q4]);  // M in the A layout
        F4 bM;                                     // M in the B layout
#pragma unroll
        for (int i = 0; i < 4; ++i) bM[i] = sm.Nd[Rd][4 * q4 + i][m16];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 eye;
#pragma unroll
        for (int i = 0; i < 4; ++i) eye[i] = (4 * q4 + i == m16) ? 1.0f : 0.0f;
        const F4 aM1 = aM, bM1 = bM;
        const F4 bM2 = O::cvt(O::mma16(aM1, bM1, z)), aM2 = O::cvt(O::mma16(bM1, aM1, z));  // M^2
        const F4 bM4 = O::cvt(O::mma16(aM2, bM2, z)), aM4 = O::cvt(O::mma16(bM2, aM2, z));  // M^4
        const f32x4 M8 = O::mma16(aM4, bM4, z);                                             // M^8
        f32x4 Y = M8 + eye;                          // I + M^8
        Y = O::mma16(aM4, O::cvt(Y), Y);             // (I + M^4)(I + M^8)
        Y = O::mma16(aM2, O::cvt(Y), Y);             // (I + M^2) ...
        Y = O::mma16(aM1, O::cvt(Y), Y);             // (I + M) ...
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.Tb[Rd][4 * q4 + i][m16] = (OT)Y[i];
    }

    // Off-diagonal block (Rr, I), I < Rr: -A (beta-scaled) and / or P
    template <bool DoA, bool DoP_>
    __device__ __forceinline__ void p2_pair(int Rr, int I)
    {
        constexpr bool DoP = DoP_ && !NoQ;
        const int pid = pair_id(Rr, I);
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 32 * s + 4 * q4;
            const float* kl = &sm.key.f.KL[16 * Rr + m16][c];
            const float* ql = &sm.key.f.QL[16 * Rr + m16][c];
            const float* ks = &sm.key.f.KS[16 * I + m16][c];
            // adjacent blocks (I = Rr - 1) have no block between them: their
            // factor 2^(rho_Rr - rho_{I+1}) is exactly 1
            const F8 b = I + 1 == Rr ? O::cat2(O::cvt(ld4f(ks)), O::cvt(ld4f(ks + 16)))
                                     : O::cat2(O::cvt(ld4f(ks) * ld4f(&sm.Fo[pid][c])),
                                               O::cvt(ld4f(ks + 16) * ld4f(&sm.Fo[pid][c + 16])));
            if (DoA) accA = O::mma32(O::cat2(O::cvt(ld4f(kl)), O::cvt(ld4f(kl + 16))), b, accA);
            if (DoP) accP = O::mma32(O::cat2(O::cvt(ld4f(ql)), O::cvt(ld4f(ql + 16))), b, accP);
            if constexpr (!Lean) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q4 + i;
            if (DoA) sm.An[pid][row][m16] = (OT)(-accA[i] * sm.beta[16 * Rr + row]);
            if (DoP) sm.Pb[tri_id(Rr, I)][row][m16] = (OT)accP[i];
        }
    }

    // P2 with 8 wavefronts: 0 .. NB-1 the diagonal blocks, the rest the
    // off-diagonal pairs. With four blocks the six pairs go to four
    // wavefronts as one pair (A and P) plus the A or the P half of one of the
    // last two pairs each; wavefronts w and w + 4 share a SIMD, so every SIMD
    // gets a diagonal block and one and a half pairs.
    __device__ __forceinline__ void p2()
    {
        constexpr int kW = kWaves;
        if (wave < NB) {
            p2_diag(wave);
        } else if constexpr (Lean && NB == 4 && kW == 8) {
            if (wave == 4) {
                p2_pair<true, true>(1, 0);
                p2_pair<true, false>(3, 1);
            } else if (wave == 5) {
                p2_pair<true, true>(2, 0);
                p2_pair<true, false>(3, 2);
            } else if (wave == 6) {
                p2_pair<true, true>(2, 1);
                p2_pair<false, true>(3, 1);
            } else {
                p2_pair<true, true>(3, 0);
                p2_pair<false, true>(3, 2);
            }
        } else {
#pragma unroll
            for (int Rr = 1; Rr < NB; ++Rr)
#pragma unroll
                for (int I = 0; I < Rr; ++I)
                    if (NB + pair_id(Rr, I) % (kW - NB) == wave) p2_pair<true, true>(Rr, I);
        }
    }

    // P2b: k o 2^b, q o 2^b over the dead float32 region. Lean: q o 2^b, and
    // the transposed right-hand sides -beta k o 2^b and beta v (each rounded
    // once to the operand type; the 8 tokens of a channel in one 16-byte store)
    __device__ __forceinline__ void p2b()
    {
        if (!prod) return;
        if constexpr (Lean) {
            static_assert(RP == 8 && !F32P, "transposed staging: 8 tokens per producer thread, float16 operands");
            h8 w0, w1, u0, u1;
#pragma unroll
            for (int t = 0; t < RP; ++t) {
                if constexpr (!NoQ) *reinterpret_cast<typename O::P2*>(&sm.key.x.Qt[rbase + t][c0]) = qt2[t];
                w0[t] = kt2[t].x;
                w1[t] = kt2[t].y;
                u0[t] = xu2[t].x;
                u1[t] = xu2[t].y;
            }
            *reinterpret_cast<h8*>(&sm.key.x.XWt[c0][rbase]) = w0;
            *reinterpret_cast<h8*>(&sm.key.x.XWt[c0 + 1][rbase]) = w1;
            *reinterpret_cast<h8*>(&sm.key.x.XUt[c0][rbase]) = u0;
            *reinterpret_cast<h8*>(&sm.key.x.XUt[c0 + 1][rbase]) = u1;
            return;
        }
#pragma unroll
        for (int t = 0; t < RP; ++t) {
            *reinterpret_cast<typename O::P2*>(&sm.key.h.Kt[rbase + t][c0]) = kt2[t];
            *reinterpret_cast<typename O::P2*>(&sm.key.h.Qt[rbase + t][c0]) = qt2[t];
        }
    }
};

}  // namespace
}  // namespace kda
