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
//   matters: the matrix-core form below (16 rows x 64 bytes per load
//   instruction) streams W at only about 3.7 TB/s, so it serves only 5 to 8
//   tokens, where the arithmetic of this form grows past it.
// * gemv_fp8_mfma_kernel: 16 rows of W per workgroup through 16x16x32 bf16
//   products (the E4M3 codes converted exactly to bf16, x's rows as the other
//   operand), float32 block partials scaled once per 128-k block.
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
// XQ: x holds E4M3 codes with per-(row, 128-column group) scales (W8A8); a
// lane's 16 values lie in one group, so each row adds one scale per step.
template <typename TOUT, int M, int R, int S, bool XQ>
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
                float xv[M][16], xsc[M];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if constexpr (XQ) {
                        decode16(ld16(static_cast<const uint8_t*>(a.x) + m * a.ldx + k), xv[m]);
                        xsc[m] = sc * a.xs[m * a.xs_ld + (k >> 7)];
                    } else {
                        const bf16_t* xp = x + m * a.ldx + k;
                        const f32x4 x0 = ld4(xp), x1 = ld4(xp + 4), x2 = ld4(xp + 8), x3 = ld4(xp + 12);
                        const float t[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                             x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
                        for (int e = 0; e < 16; ++e) xv[m][e] = t[e];
                        xsc[m] = sc;
                    }
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
                        acc[r][m] += xsc[m] * d;
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kMfmaSteps = 4;            // 128-k blocks of W (and x) in flight per wavefront
constexpr int64_t kWaveTarget = 2560;  // about ten wavefronts per compute unit, all resident at once

// 8 E4M3 codes (two dwords, lowest byte first) -> 8 bfloat16 by the hardware
// conversion with unit scale; exact, since every E4M3 value is a bfloat16
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t d0, uint32_t d1)
{
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, true);
    return bf16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Several tokens (5 to 8): the arithmetic of the form above grows with the
// token count and bounds it, so the 16-row tiles go through the matrix cores.
// One workgroup per 16 rows of W, KS wavefronts splitting its 128-k blocks
// round robin (block kb to wavefront kb % KS). Per block a lane loads 2 x 16
// codes of its row (lane % 16) at k = 16 (lane / 16) and 64 + 16 (lane / 16)
// and the same k of x's row lane % 16, so that four 16x16x32 products give the
// block's 16 x 16 partial y in float32; the block scale (staged in LDS)
// multiplies it once. The loads of the next kMfmaSteps - 1 blocks are in flight
// while a block is computed; the loop body has no branches (loads past a
// wavefront's last block re-read that block and are not accumulated), so the
// waits stay exact. The KS partial results are summed in a fixed order through
// LDS.
// XQ: x holds E4M3 codes (converted exactly to bfloat16 like W's) and its
// per-(token, block) scale joins the block scale of W.
template <typename TOUT, int KS, bool XQ>
__global__ __launch_bounds__(KS * 64) void gemv_fp8_mfma_kernel(Fp8GemvArgs a)
{
    extern __shared__ float scl[];  // the K / 128 block scales of these rows
    __shared__ f32x4 red[KS > 1 ? KS - 1 : 1][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nkb = (int)(a.K >> 7);
    const int cnt = (nkb - wave + KS - 1) / KS;  // this wavefront's blocks: wave, wave + KS, ... (at least one)
    // A lane past the last row of W or the last token reads row 0 instead: an
    // output row or column depends only on its own row of W or x, and those
    // past the ends are never stored.
    const bool xok = r16 < a.M;
    const uint8_t* wp = a.w + (n0 + r16 < a.N ? n0 + r16 : 0) * a.ldw + 16 * q4;
    const bf16_t* xp = static_cast<const bf16_t*>(a.x) + (xok ? r16 : 0) * a.ldx + 16 * q4;
    const uint8_t* xq = static_cast<const uint8_t*>(a.x) + (xok ? r16 : 0) * a.ldx + 16 * q4;
    const float* xsr = XQ ? a.xs + (xok ? r16 : 0) * a.xs_ld : nullptr;

    // x: bfloat16 (four 16-byte pieces per block) or codes (two, as W's)
    u32x4_t wb[kMfmaSteps][2], xb[kMfmaSteps][4];
#define KDA_GEMV_LOAD(T, S)                                                                         \
    {                                                                                               \
        const int64_t k_ = (int64_t)(wave + KS * min((T), cnt - 1)) * 128;                          \
        wb[S][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + k_));            \
        wb[S][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + k_ + 64));       \
        if constexpr (XQ) {                                                                         \
            xb[S][0] = ld16(xq + k_);                                                               \
            xb[S][1] = ld16(xq + k_ + 64);                                                          \
        } else {                                                                                    \
            xb[S][0] = ld16(xp + k_);                                                               \
            xb[S][1] = ld16(xp + k_ + 8);                                                           \
            xb[S][2] = ld16(xp + k_ + 64);                                                          \
            xb[S][3] = ld16(xp + k_ + 72);                                                          \
        }                                                                                           \
    }
#pragma unroll
    for (int s = 0; s < kMfmaSteps; ++s) KDA_GEMV_LOAD(s, s)
    {
        const float* sp = a.ws + (n0 >> 7) * a.ws_ld;  // 16 | 128: the rows share one block row of scales
        for (int i = threadIdx.x; i < nkb; i += KS * 64) scl[i] = sp[i];
        __syncthreads();
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < cnt; t0 += kMfmaSteps) {
#pragma unroll
        for (int s = 0; s < kMfmaSteps; ++s) {
            const int t = t0 + s;
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8_t x0 = XQ ? codes_to_bf16(xb[s][h][0], xb[s][h][1]) : __builtin_bit_cast(bf16x8_t, xb[s][2 * h]);
                const bf16x8_t x1 = XQ ? codes_to_bf16(xb[s][h][2], xb[s][h][3]) : __builtin_bit_cast(bf16x8_t, xb[s][2 * h + 1]);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(wb[s][h][0], wb[s][h][1]), x0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(wb[s][h][2], wb[s][h][3]), x1, c, 0, 0, 0);
            }
            const int kb_ = wave + KS * min(t, cnt - 1);
            const float sc = XQ ? scl[kb_] * xsr[kb_] : scl[kb_];
            const bool live = t < cnt;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = live ? fmaf(sc, c[e], acc[e]) : acc[e];
            KDA_GEMV_LOAD(t + kMfmaSteps, s)
        }
    }
#undef KDA_GEMV_LOAD
    // lane (j, q) holds y[token j][rows n0 + 4q .. n0 + 4q + 3]
    if constexpr (KS > 1) {
        if (wave > 0) red[wave - 1][lane] = acc;
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < KS - 1; ++w) acc += red[w][lane];
    }
    if (xok) {
        TOUT* y = static_cast<TOUT*>(a.y) + r16 * a.ldy;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t n = n0 + 4 * q4 + e;
            if (n < a.N) st(y + n, acc[e]);
        }
    }
}

template <typename T> __device__ __forceinline__ f32x2 ld2_nt(const T* p);
template <> __device__ __forceinline__ f32x2 ld2_nt<float>(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
}
template <> __device__ __forceinline__ f32x2 ld2_nt<bf16_t>(const bf16_t* p)
{
    const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
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
    // o and the gate columns are read once: non-temporal, as in the bf16
    // epilogue, so that the codes the output projection reads next stay cached
    const f32x2 ov = ld2_nt(static_cast<const TO*>(a.o) + row * 128 + c);
    const float ms = wave_sum(ov.x * ov.x + ov.y * ov.y) * (1.0f / 128.0f);
    const float r = rsqrtf(ms + a.eps);
    const f32x2 gv = ld2_nt(static_cast<const TG*>(a.gate) + t * a.gate_ld + (int64_t)h * 128 + c);
    const float y0 = ov.x * r * a.w[c] * sigmoidf_(gv.x);
    const float y1 = ov.y * r * a.w[c + 1] * sigmoidf_(gv.y);
    const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0 / scale, y1 / scale, 0, false);
    *reinterpret_cast<uint16_t*>(a.codes + row * 128 + c) = (uint16_t)(packed & 0xffff);
    if (lane == 0) a.scales[row] = scale;
}


// ------------------------------------------------ activation quantization
// One wavefront per 512 columns of a row: a lane takes 8 consecutive values,
// so each 16-lane row of the wavefront holds one 128-column group, whose
// maximum magnitude is a 16-lane reduction. Every rounding step is float32:
// scale = amax / 448 and x / scale by correctly rounded division, the
// quotient clamped to +-448 (a quotient a hair above 448 stays on the largest
// code) and converted to E4M3 with ties to even by the hardware conversion.
template <typename TX>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(QuantFp8Args a)
{
    const int lane = threadIdx.x & 63;
    const int64_t strips = (a.K + 511) / 512;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= a.M * strips) return;
    const int64_t m = wid / strips;
    const int64_t k = (wid % strips) * 512 + 8 * lane;
    const bool in = k < a.K;  // K is a multiple of 128: whole groups are in or out
    float v[8];
    if (in) {
        const TX* xp = static_cast<const TX*>(a.x) + m * a.ldx + k;
        if constexpr (sizeof(TX) == 2) {
            Vec16<bf16_t>::unpack(ld16(xp), v);
        } else {
            Vec16<float>::unpack(ld16(xp), v);
            Vec16<float>::unpack(ld16(xp + 4), v + 4);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
    am = group_max<16>(am);
    const float scale = am > 0.f ? __fdiv_rn(am, 448.0f) : 1.0f;
    if (!in) return;
    uint32_t w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = fminf(fmaxf(__fdiv_rn(v[4 * d + e], scale), -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], p, true);
        w[d] = (uint32_t)p;
    }
    *reinterpret_cast<uint2*>(a.codes + m * a.ldc + k) = make_uint2(w[0], w[1]);
    if ((lane & 15) == 0) a.scales[m * a.lds + (k >> 7)] = scale;
}

// ---------------------------------------------------------- W8A8 GEMM
// Y[M, N] = X W^T, both operands block FP8 (X per row and 128-column group,
// W per 128 x 128 block). A workgroup of eight wavefronts computes a 256 x 256
// tile of Y, a wavefront 64 rows of X by 128 rows of W (one block row of W's
// scales). K runs in steps of one 128-wide scale block, double-buffered in
// LDS by buffer-to-LDS copies: per step and 16 x 16 tile one 16x16x128 FP8
// matrix product from zero (the E4M3 products are exact and summed in
// float32), then acc += (sx[row, kb] * sw[n / 128, kb]) * P on the vector
// unit, which runs beside the matrix unit. Rows are 128 bytes in LDS with
// their 16-byte chunks XOR-swizzled by row mod 8 (the swizzle is applied
// through each lane's source address), so that the rows of an operand read
// spread over the banks. As in the bf16 GEMM, the product is formed
// transposed, so that a lane holds four consecutive columns of one row of Y.
// Per block a wavefront issues the eight products of two W tiles and its four
// X tiles into separate registers before scaling them in, so that the matrix
// unit runs while the vector unit adds (one shared result register left every
// product's latency exposed).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int kF8Tile = 256;                  // rows of X and of W per workgroup
constexpr int kF8Stage = 2 * kF8Tile * 128;   // one K step: X rows, then W rows
typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte chunk c (0..7) of row r: slot c ^ ((r / 2) mod 8). A fragment read
// takes one chunk of 16 consecutive rows; rows r and r + 1 fall in different
// halves of the 64 banks and the even (odd) rows of the 16 get distinct slots,
// so the read is free of bank conflicts (with slot c ^ (r mod 8), rows r and
// r + 8 collided: 2-way conflicts on every read).
__device__ __forceinline__ int swz8(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <typename TC, bool VEC>
__global__ __launch_bounds__(512) void gemm_fp8_kernel(Fp8GemvArgs a)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][kF8Stage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
    const int64_t tiles_m = (a.M + kF8Tile - 1) / kF8Tile;
    const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int64_t m0 = tm * kF8Tile, n0 = tn * kF8Tile;

    // rows past M or N read as zero through the descriptor ranges
    const uint8_t* X = static_cast<const uint8_t*>(a.x) + m0 * a.ldx;
    const uint8_t* Wr = a.w + n0 * a.ldw;
    const int64_t rows_x = min<int64_t>(kF8Tile, a.M - m0), rows_w = min<int64_t>(kF8Tile, a.N - n0);
    const rsrc_t rx = make_rsrc(X, (rows_x - 1) * a.ldx + a.K);
    const rsrc_t rw = make_rsrc(Wr, (rows_w - 1) * a.ldw + a.K);

    // copy of K step kb into stage st: 64 instructions of 1 KiB, 8 per
    // wavefront (X rows for waves 0-3, W rows for 4-7); instruction j of a
    // wavefront covers rows 64 (wave mod 4) + 8 j + l / 8 (lane l) into LDS
    // chunk slot l % 8, which holds K chunk slot ^ ((row / 2) mod 8). That
    // swizzle depends on j only through its parity, so two lane offsets serve
    // all eight instructions and the row step 8 j ld goes into the scalar offset
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)&smem[0][0];
    const bool cw = wave >= 4;
    const rsrc_t rc = cw ? rw : rx;
    const int ldc = (int)(cw ? a.ldw : a.ldx);
    const int rb = 64 * (wave & 3) + (lane >> 3);
    int voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) voff[par] = rb * ldc + 16 * ((lane & 7) ^ (((rb >> 1) + 4 * par) & 7));
    auto copy = [&](int kb, int st, int j0, int j1) {
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const uint32_t dst = lds0 + st * kF8Stage + (wave * 8 + j) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void_t*)(uintptr_t)dst, 16, voff[j & 1], 8 * j * ldc + kb * 128, 0, 0);
        }
    };

    // scales: this lane's four rows of X, and the block row of W of this wavefront
    const float* sxp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = m0 + wm + 16 * i + m16;
        sxp[i] = a.xs + (r < a.M ? r : a.M - 1) * a.xs_ld;
    }
    const int64_t wb_row = (n0 + wn) >> 7, wb_last = (a.N - 1) >> 7;
    const float* swp = a.ws + (wb_row < wb_last ? wb_row : wb_last) * a.ws_ld;

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the scales of step kb + 1 are loaded one step ahead, before that step's
    // copy: a load issued after the copy would make its first use wait for
    // the copy as well (the vector memory counter drains in order), which
    // stalled every step on the next step's copy
    float sxv[4], swv;
    auto load_scales = [&](int kb) {
        swv = swp[kb];
#pragma unroll
        for (int i = 0; i < 4; ++i) sxv[i] = sxp[i][kb];
    };
    const int nk = (int)(a.K >> 7);
    load_scales(0);
    copy(0, 0, 0, 8);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's copy has landed
    __syncthreads();
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < nk; ++kb) {
        const int st = kb & 1;
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = sxv[i] * swv;
        if (kb + 1 < nk) {
            load_scales(kb + 1);
            copy(kb + 1, st ^ 1, 0, 8);
        }
        const uint8_t* sa = &smem[st][0];
        const uint8_t* sb = &smem[st][kF8Tile * 128];
        i32x8_t fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm + 16 * i + m16;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sa + swz8(r, 2 * q4));
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sa + swz8(r, 2 * q4 + 1));
            fa[i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            i32x8_t fb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn + 16 * (2 * h + j) + m16;
                const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sb + swz8(r, 2 * q4));
                const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sb + swz8(r, 2 * q4 + 1));
                fb[j] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            f32x4 p[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    // formats 0 / 0: E4M3 operands; block scales 127 (E8M0 1.0)
                    p[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], fa[i], zero, 0, 0, 0, 127, 0, 127);
            // the eight products first, then the 32 scale-adds
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x4& c = acc[i][2 * h + j];
#pragma unroll
                    for (int e = 0; e < 4; ++e) c[e] = fmaf(p[i][j][e], s[i], c[e]);
                }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's copy of step kb + 1 has landed
        __syncthreads();  // every copy of step kb + 1 has landed and every read of stage st is done
    }

    // acc[i][j]: lane (m16, q4) element e is Y[row 16i + m16][column 16j + 4q4 + e]
    TC* Y = static_cast<TC*>(a.y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm + 16 * i + m16;
        if (row >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t col = n0 + wn + 16 * j + 4 * q4;
            TC* p = Y + row * a.ldy + col;
            if (VEC && col + 3 < a.N) {
                st4(p, acc[i][j]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < a.N) st(p + e, acc[i][j][e]);
            }
        }
    }
}
}  // namespace

template <int M, int R, int S>
void launch_gemv_rs(const Fp8GemvArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.N + kWaves * R - 1) / (kWaves * R))), block(kWaves * 64);
    if (a.xs) {
        if (a.y_dtype == F32) hipLaunchKernelGGL((gemv_fp8_kernel<float, M, R, S, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemv_fp8_kernel<bf16_t, M, R, S, true>), grid, block, 0, s, a);
    } else {
        if (a.y_dtype == F32) hipLaunchKernelGGL((gemv_fp8_kernel<float, M, R, S, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemv_fp8_kernel<bf16_t, M, R, S, false>), grid, block, 0, s, a);
    }
}

static void launch_gemv_mfma(const Fp8GemvArgs& a, hipStream_t s)
{
    // split K over up to 8 wavefronts per 16 rows while the whole grid stays
    // within about ten wavefronts per compute unit (one round, no tail)
    const int64_t tiles = (a.N + 15) / 16;
    const int64_t nkb = a.K / 128;
    int ks = 1;
    while (ks < 8 && 2 * ks <= nkb && tiles * 2 * ks <= kWaveTarget) ks *= 2;
    const dim3 grid((unsigned)tiles), block(64 * ks);
    const size_t lds = (size_t)nkb * sizeof(float);
#define KDA_GEMV_CASE(KS)                                                                                         \
    case KS:                                                                                                      \
        if (a.xs) {                                                                                               \
            if (a.y_dtype == F32) hipLaunchKernelGGL((gemv_fp8_mfma_kernel<float, KS, true>), grid, block, lds, s, a); \
            else hipLaunchKernelGGL((gemv_fp8_mfma_kernel<bf16_t, KS, true>), grid, block, lds, s, a);              \
        } else {                                                                                                  \
            if (a.y_dtype == F32) hipLaunchKernelGGL((gemv_fp8_mfma_kernel<float, KS, false>), grid, block, lds, s, a); \
            else hipLaunchKernelGGL((gemv_fp8_mfma_kernel<bf16_t, KS, false>), grid, block, lds, s, a);             \
        }                                                                                                         \
        break;
    switch (ks) {
        KDA_GEMV_CASE(1) KDA_GEMV_CASE(2) KDA_GEMV_CASE(4) KDA_GEMV_CASE(8)
    }
#undef KDA_GEMV_CASE
}

hipError_t launch_gemv_fp8(const Fp8GemvArgs& a, hipStream_t s)
{
    // measured on the 41,024 x 4,096 projection: one token, 2 rows per
    // wavefront with 4 KiB of each in flight (29.2 us; 4 rows x 1 KiB 30.7);
    // two tokens, 2 rows x 2 KiB (32.0 us; 4 x 1 KiB 34.2); three or four,
    // 4 rows x 1 KiB, so that x's values serve 4 rows (4 tokens 42.9 us); 5 to
    // 8 tokens, the matrix-core form, whose cost hardly grows with the token
    // count (8 tokens: the 4 x 1 KiB form took 79.7 us)
    switch (a.M) {
        case 1: launch_gemv_rs<1, 2, 4>(a, s); break;
        case 2: launch_gemv_rs<2, 2, 2>(a, s); break;
        case 3: launch_gemv_rs<3, 4, 1>(a, s); break;
        case 4: launch_gemv_rs<4, 4, 1>(a, s); break;
        case 5: case 6: case 7: case 8: launch_gemv_mfma(a, s); break;
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

hipError_t launch_quantize_fp8(const QuantFp8Args& a, hipStream_t s)
{
    const int64_t waves = a.M * ((a.K + 511) / 512);
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (a.x_dtype == F32) hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(quantize_fp8_kernel<bf16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const Fp8GemvArgs& a, hipStream_t s)
{
    const int64_t tiles = ((a.M + kF8Tile - 1) / kF8Tile) * ((a.N + kF8Tile - 1) / kF8Tile);
    const dim3 grid((unsigned)tiles), block(512);
    const size_t ysz = a.y_dtype == F32 ? 4 : 2;
    const bool vec = a.ldy % 4 == 0 && (uintptr_t)a.y % (4 * ysz) == 0;
    if (a.y_dtype == F32) {
        if (vec) hipLaunchKernelGGL((gemm_fp8_kernel<float, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_fp8_kernel<float, false>), grid, block, 0, s, a);
    } else {
        if (vec) hipLaunchKernelGGL((gemm_fp8_kernel<bf16_t, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_fp8_kernel<bf16_t, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
