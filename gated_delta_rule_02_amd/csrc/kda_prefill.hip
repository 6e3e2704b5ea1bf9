// kda_prefill.hip -- chunked KDA prefill over packed sequences on gfx950 MFMA.
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
// Every factor 2^x of a block product then lies in [2^-116, 2^116] because the
// log-retention is clamped at -5 ("safe forget gate ... lower bound -5" in the
// flozi.net section above): 15 tokens x 5 x log2(e) < 116 < 127.
//
// Work split. A workgroup (4 wavefronts) owns one (sequence, head, 64 value
// columns); wavefront w owns 16 columns and keeps its 128 x 16 float32 slice
// of the state in registers for the whole sequence (value columns of the state
// evolve independently). Per chunk:
//   P0  each thread (2 key channels, one 16-token block) sums its block's
//       log-retention; the block totals are exchanged through LDS.
//   P1  the same thread forms the decay factors by running products of
//       alpha = 2^g and writes the key-side operands k o 2^l, q o 2^l, k o 2^s
//       (float32) and the transposed K-bar (float16); it keeps k o 2^b and
//       q o 2^b (float16) in registers.
//   P2  each wavefront computes some 16 x 16 blocks of A and P on MFMA and
//       one diagonal-block inverse.
//   P2b the float32 region is dead: k o 2^b and q o 2^b are written over it.
//   P3  every wavefront runs its own value-side chain (X, block forward
//       substitution, O, state update) on MFMA with no further barrier.
// The next chunk's inputs are loaded into registers while a chunk computes.
// Workgroups of one head are mapped to the same XCD so that the second one
// finds q, k, g in that XCD's L2.
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
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int D = 128;        // dk = dv
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kDvBlock = 16 * kWaves;  // value columns per workgroup
constexpr int kDvBlocks = D / kDvBlock;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- MFMA ops
// Operand layout of the 16 x 16 MFMAs used here. A K16 slab: lane
// (m = lane % 16, q = lane / 16) holds A[m][4q..4q+3] and B[4q..4q+3][n = m];
// the 16 x 16 result holds C[4q+i][n] in element i. A K32 step concatenates
// two K16 slabs per lane (elements 0-3 from the first, 4-7 from the second);
// A and B use the same assignment, so the product sums every k exactly once.
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

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
    // A K16 step runs as the K32 instruction with a zero second half: dependent
    // chains that mixed the 16x16x16 and 16x16x32 forms returned stale
    // accumulator elements on gfx950, so only the K32 form is used.
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
};

// Two consecutive input elements kept raw in a register between load and use.
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
    using type = uint32_t;
    __device__ static f32x2 unpack(uint32_t u) { return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)}; }
};
template <> struct Pair<float> {
    using type = uint2;
    __device__ static f32x2 unpack(uint2 u) { return f32x2{__uint_as_float(u.x), __uint_as_float(u.y)}; }
};
template <typename T>
__device__ __forceinline__ typename Pair<T>::type ldpair(const T* p)
{
    return *reinterpret_cast<const typename Pair<T>::type*>(p);
}
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }

// index of the off-diagonal block pair (R, I), I < R
__host__ __device__ constexpr int pair_id(int R, int I) { return R * (R - 1) / 2 + I; }
// index of the lower-triangle block (R, I), I <= R
__host__ __device__ constexpr int tri_id(int R, int I) { return R * (R + 1) / 2 + I; }

template <bool F32P>
struct __attribute__((aligned(16))) Smem {
    using OT = typename Ops<F32P>::OT;
    static constexpr int C = Ops<F32P>::C;
    static constexpr int NB = C / 16;
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr int LDK = D + 4;               // row stride of the float32 [C][128] arrays
    static constexpr int LDH = D + Ops<F32P>::PAD;  // row stride of the operand-type [C][128] arrays
    static constexpr int LDT = C + Ops<F32P>::PAD;  // row stride of [128][C]
    // P1 -> P2: key-side operands in float32. Their factors span 2^-116 .. 1
    // and the diagonal blocks rescale them by up to 2^116, beyond float16's
    // range, so each use rounds once to the MFMA operand type.
    // P2b -> P3: the same bytes then hold k o 2^b and q o 2^b (operand type).
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
    } key;
    OT KbT[D][LDT];                         // (k o 2^(b_C - b))^T   (state update)
    OT Nd[NB][16][16];                      // -A diagonal blocks (strictly lower, beta-scaled)
    OT Tb[NB][16][16];                      // (I + A_RR)^-1
    OT An[NPAIR > 0 ? NPAIR : 1][16][16];   // -A off-diagonal blocks (beta-scaled)
    OT Pb[NB * (NB + 1) / 2][16][16];       // P lower-triangle blocks
    float Fd[NB][D];                        // 2^-G_R
    float Fo[NPAIR > 0 ? NPAIR : 1][D];     // 2^(rho_R - rho_{I+1})
    float Gt[NB][D];                        // block totals of the log-retention (base 2)
    float bC[D];                            // 2^b_C
    float beta[C];
};

template <bool F32P, typename TIN, typename TOUT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a)
{
    using O = Ops<F32P>;
    using OT = typename O::OT;
    using F4 = typename O::F4;
    using F8 = typename O::F8;
    using SM = Smem<F32P>;
    constexpr int C = SM::C;
    constexpr int NB = SM::NB;

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m16 = lane & 15;
    const int q4 = lane >> 4;

    // XCD-aware order: consecutive logical ids (the value blocks of one head)
    // land on the same XCD (workgroups are dealt round-robin over 8 XCDs).
    int bid = blockIdx.x;
    if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const int dvblk = bid % kDvBlocks;
    bid /= kDvBlocks;
    const int h = bid % a.H;
    const int n = bid / a.H;
    const int jcol = dvblk * kDvBlock + wave * 16 + m16;  // this lane's value column

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

    const int64_t tok_stride = (int64_t)a.H * D;
    const TIN* qg = static_cast<const TIN*>(a.q) + (int64_t)h * D;
    const TIN* kg = static_cast<const TIN*>(a.k) + (int64_t)h * D;
    const TIN* gg = static_cast<const TIN*>(a.g) + (int64_t)h * D;
    const TIN* vg = static_cast<const TIN*>(a.v) + (int64_t)h * D + jcol;
    const TIN* bg = static_cast<const TIN*>(a.beta) + h;
    TOUT* og = static_cast<TOUT*>(a.o) + (int64_t)h * D + jcol;
    const float lbl = a.lower_bound * kLog2e;

    // Raw inputs of one chunk, loaded one chunk ahead. Rows past the end of
    // the sequence load a valid row (clamped) and are zeroed on use, so every
    // load is unconditional and all of them are in flight together.
    using PT = typename Pair<TIN>::type;
    const int R = wave;       // P0/P1 token block of this thread
    const int c0 = 2 * lane;  // P0/P1 key channels c0, c0 + 1
    PT rk[16], rq[16], rg[16];
    TIN rv[NB][4];            // v[16R' + 4q + i][jcol]
    TIN rb = TIN(0);
    const int ts32 = a.H * D;  // token stride in elements (fits 32 bits)
    auto load_kqg = [&](int64_t c_s, int nt) {  // consumed in P0/P1
        const int64_t base = c_s * tok_stride;
        if (R < NB) {
            const TIN *kb_ = kg + base, *qb_ = qg + base, *gb_ = gg + base;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int off = min(16 * R + rr, nt - 1) * ts32 + c0;
                rk[rr] = ldpair(kb_ + off);
                rq[rr] = ldpair(qb_ + off);
                rg[rr] = ldpair(gb_ + off);
            }
        }
        if (tid < C) rb = bg[(c_s + min(tid, nt - 1)) * a.H];
    };
    auto load_v = [&](int64_t c_s, int nt) {  // consumed in P3
        const TIN* vb_ = vg + c_s * tok_stride;
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr)
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[Rr][i] = vb_[min(16 * Rr + 4 * q4 + i, nt - 1) * ts32];
    };
    if (seq_s < seq_e) {
        load_kqg(seq_s, (int)min<int64_t>(C, seq_e - seq_s));
        load_v(seq_s, (int)min<int64_t>(C, seq_e - seq_s));
    }

    for (int64_t cs = seq_s; cs < seq_e; cs += C) {
        const int ntok = (int)min<int64_t>(C, seq_e - cs);

        // ---------------- P0: block totals of the log-retention (base 2)
        f32x2 g2[16];
        if (R < NB) {
            f32x2 G = {0.f, 0.f};
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const f32x2 gv = Pair<TIN>::unpack(rg[rr]);
                const bool valid = 16 * R + rr < ntok;
                g2[rr] = valid ? f32x2{fmaxf(gv.x * kLog2e, lbl), fmaxf(gv.y * kLog2e, lbl)} : f32x2{0.f, 0.f};
                G += g2[rr];
            }
            *reinterpret_cast<f32x2*>(&sm.Gt[R][c0]) = G;
        }
        if (tid < C) sm.beta[tid] = tid < ntok ? to_f32(rb) : 0.0f;
        __syncthreads();

        // ---------------- P1: decay factors and key-side operands
        // kt/qt: k o 2^b and q o 2^b in the operand type, written in P2b
        F4 kt[8], qt[8];
        if (R < NB) {
            f32x2 rho_R = {0.f, 0.f}, rho_R1, bCv = {0.f, 0.f};
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                const f32x2 gJ = *reinterpret_cast<const f32x2*>(&sm.Gt[J][c0]);
                if (J < R) rho_R += gJ;
                bCv += gJ;
            }
            const f32x2 GR = *reinterpret_cast<const f32x2*>(&sm.Gt[R][c0]);
            rho_R1 = rho_R + GR;
            // factor tables for P2 and P3 (this thread's two channels)
            *reinterpret_cast<f32x2*>(&sm.Fd[R][c0]) = f32x2{exp2_fast(-GR.x), exp2_fast(-GR.y)};
            {
                f32x2 rho_I1 = {0.f, 0.f};
#pragma unroll
                for (int I = 0; I < NB - 1; ++I) {
                    rho_I1 += *reinterpret_cast<const f32x2*>(&sm.Gt[I][c0]);
                    if (I < R)  // pair (R, I): index R (R - 1) / 2 + I
                        *reinterpret_cast<f32x2*>(&sm.Fo[R * (R - 1) / 2 + I][c0]) =
                            f32x2{exp2_fast(rho_R.x - rho_I1.x), exp2_fast(rho_R.y - rho_I1.y)};
                }
            }
            if (R == 0) *reinterpret_cast<f32x2*>(&sm.bC[c0]) = f32x2{exp2_fast(bCv.x), exp2_fast(bCv.y)};
            const f32x2 DR = {exp2_fast(rho_R.x), exp2_fast(rho_R.y)};
            const f32x2 fb = {exp2_fast(bCv.x - rho_R1.x), exp2_fast(bCv.y - rho_R1.y)};

            // forward: e_l = prod_{j<=r} alpha_j ; reverse: e_s = prod_{j>r} alpha_j
            f32x2 al[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) al[rr] = f32x2{exp2_fast(g2[rr].x), exp2_fast(g2[rr].y)};
            f32x2 el = {1.f, 1.f};
            f32x4 k4[2], q4v[2];  // 4 tokens of k o 2^b / q o 2^b per channel
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const bool valid = 16 * R + rr < ntok;
                el *= al[rr];
                f32x2 kv = Pair<TIN>::unpack(rk[rr]), qv = Pair<TIN>::unpack(rq[rr]);
                kv = valid ? kv : f32x2{0.f, 0.f};
                qv = valid ? qv : f32x2{0.f, 0.f};
                const int r = 16 * R + rr;
                const f32x2 klv = kv * el, qlv = qv * el;
                *reinterpret_cast<f32x2*>(&sm.key.f.KL[r][c0]) = klv;
                *reinterpret_cast<f32x2*>(&sm.key.f.QL[r][c0]) = qlv;
                const f32x2 ktt = klv * DR, qtt = qlv * DR;
                k4[0][rr & 3] = ktt.x; k4[1][rr & 3] = ktt.y;
                q4v[0][rr & 3] = qtt.x; q4v[1][rr & 3] = qtt.y;
                if ((rr & 3) == 3) {  // kt[4e + j]: channel c0 + e, tokens 16R + 4j .. +3
                    kt[rr >> 2] = O::cvt(k4[0]);
                    kt[4 + (rr >> 2)] = O::cvt(k4[1]);
                    qt[rr >> 2] = O::cvt(q4v[0]);
                    qt[4 + (rr >> 2)] = O::cvt(q4v[1]);
                }
            }
            f32x2 es = {1.f, 1.f};
            f32x4 kb4[2];
#pragma unroll
            for (int rr = 15; rr >= 0; --rr) {
                const bool valid = 16 * R + rr < ntok;
                f32x2 kv = Pair<TIN>::unpack(rk[rr]);
                kv = valid ? kv : f32x2{0.f, 0.f};
                const f32x2 ksv = kv * es;
                *reinterpret_cast<f32x2*>(&sm.key.f.KS[16 * R + rr][c0]) = ksv;
                kb4[0][rr & 3] = ksv.x * fb.x;
                kb4[1][rr & 3] = ksv.y * fb.y;
                if ((rr & 3) == 0) {  // transposed K-bar: row = channel, tokens 16R + rr .. +3
                    *reinterpret_cast<F4*>(&sm.KbT[c0][16 * R + rr]) = O::cvt(kb4[0]);
                    *reinterpret_cast<F4*>(&sm.KbT[c0 + 1][16 * R + rr]) = O::cvt(kb4[1]);
                }
                es *= al[rr];
            }
        }
        // the next chunk's key-side inputs stream in while this chunk computes
        if (cs + C < seq_e) load_kqg(cs + C, (int)min<int64_t>(C, seq_e - cs - C));
        __syncthreads();

        // ---------------- P2: blocks of A and P, diagonal inverses
        if (wave < NB) {
            const int Rd = wave;
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
                accP = O::diagP(ld4f(ql), ld4f(ql + 16), x0, x1, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * q4 + i;  // row in block, column m16
                const float b = sm.beta[16 * Rd + row];
                sm.Nd[Rd][row][m16] = (OT)(row > m16 ? -accA[i] * b : 0.0f);
                sm.Pb[tri_id(Rd, Rd)][row][m16] = (OT)(row >= m16 ? accP[i] : 0.0f);
            }
            // wavefront-local: the inverse below reads what this wavefront wrote
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
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
        }
        // off-diagonal pairs, spread over the wavefronts
#pragma unroll
        for (int Rr = 1; Rr < NB; ++Rr)
#pragma unroll
            for (int I = 0; I < Rr; ++I) {
                const int pid = pair_id(Rr, I);
                if (pid % kWaves != wave) continue;
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int c = 32 * s + 4 * q4;
                    const float* kl = &sm.key.f.KL[16 * Rr + m16][c];
                    const float* ql = &sm.key.f.QL[16 * Rr + m16][c];
                    const float* ks = &sm.key.f.KS[16 * I + m16][c];
                    const F8 b = O::cat2(O::cvt(ld4f(ks) * ld4f(&sm.Fo[pid][c])),
                                         O::cvt(ld4f(ks + 16) * ld4f(&sm.Fo[pid][c + 16])));
                    accA = O::mma32(O::cat2(O::cvt(ld4f(kl)), O::cvt(ld4f(kl + 16))), b, accA);
                    accP = O::mma32(O::cat2(O::cvt(ld4f(ql)), O::cvt(ld4f(ql + 16))), b, accP);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * q4 + i;
                    sm.An[pid][row][m16] = (OT)(-accA[i] * sm.beta[16 * Rr + row]);
                    sm.Pb[tri_id(Rr, I)][row][m16] = (OT)accP[i];
                }
            }
        __syncthreads();

        // ---------------- P2b: k o 2^b, q o 2^b over the dead float32 region
        if (R < NB) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * R + 4 * j + i;
                    sm.key.h.Kt[r][c0] = kt[j][i];
                    sm.key.h.Kt[r][c0 + 1] = kt[4 + j][i];
                    sm.key.h.Qt[r][c0] = qt[j][i];
                    sm.key.h.Qt[r][c0 + 1] = qt[4 + j][i];
                }
        }
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
                const int r = 16 * Rr + 4 * q4 + i;
                const float vv = r < ntok ? to_f32(rv[Rr][i]) : 0.0f;
                X[Rr][i] = sm.beta[r] * (vv - accX[i]);
            }
            O1[Rr] = accO;
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
        // outputs O_R = scale (O1_R + sum_{I<=R} P_RI U_I)
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr) {
            f32x4 acc = O1[Rr];
#pragma unroll
            for (int I = 0; I + 1 <= Rr; I += 2)
                acc = O::mma32(O::cat2(O::lds(&sm.Pb[tri_id(Rr, I)][m16][4 * q4]), O::lds(&sm.Pb[tri_id(Rr, I + 1)][m16][4 * q4])),
                               O::cat2(UB[I], UB[I + 1]), acc);
            if (!(Rr & 1)) acc = O::mma16(O::lds(&sm.Pb[tri_id(Rr, Rr)][m16][4 * q4]), UB[Rr], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * Rr + 4 * q4 + i;
                if (r < ntok) st(og + (cs + r) * tok_stride, a.scale * acc[i]);
            }
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
        if (cs + C < seq_e) load_v(cs + C, (int)min<int64_t>(C, seq_e - cs - C));
        __syncthreads();
    }

    if (a.sT) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.sT[sbase + (size_t)(16 * t + 4 * q4 + i) * D + jcol] = S[t][i];
    }
}

template <bool F32P, typename TIN>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.H * kDvBlocks)), block(kThreads);
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
