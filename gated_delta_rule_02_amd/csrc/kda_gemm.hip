// kda_gemm.hip -- C[M,N] = A[M,K] B[N,K]^T, bfloat16 inputs, float32 accumulate.
//
// The token mixer's dense projections ("Ling-3.1-flash: a 560B hybrid-attention
// MoE, counted from its safetensors headers", section "How KDA and MLA split the
// work": q, k, v, decay and gate 4096 -> 8192 and the output 8192 -> 4096, all
// full rank). Both operands are K-contiguous, which is exactly the layout the
// 16x16x32 bf16 MFMA consumes: each lane takes 8 consecutive K values of one
// row of A and one row of B.
//
// Two kernels. The main one (K a multiple of 64): a 256 x 256 tile of C per
// workgroup of 4 wavefronts, each owning 128 x 128 (8 x 8 MFMA tiles, 256
// accumulator registers: one wavefront per SIMD), K steps of 64 in two LDS
// stages filled by buffer-to-LDS copies of whole 128-byte operand rows (the
// copy of step k + 1 runs during step k). With K steps of 32 every copy
// request covered half a cache line, and the kernel issued twice the L2 read
// requests of the vendor BLAS for the same product; at the per-compute-unit
// limit on requests in flight that halved its operand bandwidth. The stage
// rows are 128 bytes with their 16-byte chunks XOR-swizzled by (row / 2) mod
// 8 (applied by choosing each lane's global source address: a buffer-to-LDS
// copy writes lane l to byte 16 l of its 1 KiB destination), so that the 16
// rows an MFMA operand read touches fall in distinct banks. The products are
// formed transposed (B tile x A tile^T): each lane then holds four
// consecutive columns of one row of C, stored with one 16-byte (float32) or
// 8-byte (bfloat16) access.
// The fallback (any K multiple of 8): 128 x 128 tiles, 2 x 2 wavefronts of
// 64 x 64, K steps of 32 through double-buffered LDS.
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

// ------------------------------------------------------------ main kernel
constexpr int TM = 256, TN = 256, TK = 64;  // workgroup tile and K step (128 bytes of each operand row)
constexpr int kStageBytes = TM * TK * 2;     // one operand's stage: 256 rows x 128 B
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of 16-byte chunk c (0..7) of row r of a stage: the chunks are
// XOR-swizzled by (r / 2) mod 8. An operand read takes one chunk of 16
// consecutive rows; rows r and r + 1 lie in different halves of the 64
// banks and the 8 even (odd) rows get distinct slots, so the read touches
// every bank once.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// NJ: 16-column MFMA tiles per wavefront in N (8: the 256 x 256 tile; 2 or 4:
// a 256 x 64 or 256 x 128 tile for the last N mod 256 columns, so that they
// cost a fraction of a full tile instead of a whole one)
template <typename TC, int NJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm256_kernel(GemmArgs a)
{
    constexpr int TNW = 32 * NJ;         // columns of C per workgroup
    constexpr int kACopy = TM / 32;      // A copy instructions per wavefront and K step (8 rows each)
    constexpr int kBCopy = TNW / 32;     // B copy instructions per wavefront and K step
    static_assert(NJ == 2 || NJ == 4 || NJ == 8, "64, 128 or 256 columns");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][kStageBytes];  // [stage][A, B]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int wm = (wave >> 1) * 128, wn = (wave & 1) * 16 * NJ;

    // tiles: consecutive workgroup ids run down a column of M tiles, so the
    // workgroups resident together share B tiles and a few A tiles
    const int tiles_m = (int)((a.M + TM - 1) / TM);
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int64_t m0 = (int64_t)tm * TM, n0 = (int64_t)tn * TNW;

    // operand rows past M or N read as zero through the descriptor ranges
    const bf16_t* A = static_cast<const bf16_t*>(a.A) + m0 * a.lda;
    const bf16_t* B = static_cast<const bf16_t*>(a.B) + n0 * a.ldb;
    const int64_t rows_a = min<int64_t>(TM, a.M - m0), rows_b = min<int64_t>(TNW, a.N - n0);
    const rsrc_t ra = make_rsrc(A, ((rows_a - 1) * a.lda + a.K) * 2);
    const rsrc_t rb = make_rsrc(B, ((rows_b - 1) * a.ldb + a.K) * 2);

    // copy of K step kt into stage st: whole 128-byte rows, 8 rows per 1 KiB
    // instruction (lane l: row 8i + l/8, LDS chunk slot l%8, which holds the
    // row's K chunk slot ^ ((row / 2) mod 8))
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)&smem[0][0][0];
    const int lrow = lane >> 3, lslot = lane & 7;
    auto copy = [&](int kt, int st) {
#pragma unroll
        for (int j = 0; j < kACopy; ++j) {
            const int i = wave * kACopy + j;
            const int row = 8 * i + lrow;
            const int koff = (kt * TK + (lslot ^ ((row >> 1) & 7)) * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(uintptr_t)(lds0 + (st * 2 + 0) * kStageBytes + i * 1024),
                                                     16, (int)(row * a.lda * 2) + koff, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kBCopy; ++j) {
            const int i = wave * kBCopy + j;
            const int row = 8 * i + lrow;
            const int koff = (kt * TK + (lslot ^ ((row >> 1) & 7)) * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(uintptr_t)(lds0 + (st * 2 + 1) * kStageBytes + i * 1024),
                                                     16, (int)(row * a.ldb * 2) + koff, 0, 0, 0);
        }
    };

    f32x4 acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Pipeline: two stages of 64 K. Step kt computes on stage kt % 2 (two K32
    // halves) while the copy of step kt + 1, issued at its start, fills the
    // other stage; the second half's fragments are read while the first half's
    // MFMAs run. At its end every wavefront waits for its copy (the compiler
    // does not track these copies: the wait is explicit) and the barrier
    // hands the stage over.
    const int nk = (int)(a.K / TK);
    u32x4_t fa[8], fb[NJ];
    auto read_a = [&](int st, int h, int i) {
        fa[i] = *reinterpret_cast<const u32x4_t*>(&smem[st][0][0] + swz(wm + 16 * i + m16, 4 * h + q4));
    };
    auto read_b = [&](int st, int h, int j) {
        fb[j] = *reinterpret_cast<const u32x4_t*>(&smem[st][1][0] + swz(wn + 16 * j + m16, 4 * h + q4));
    };
    copy(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    lds_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) copy(kt + 1, st ^ 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) read_a(st, 0, i);
#pragma unroll
        for (int j = 0; j < NJ; ++j) read_b(st, 0, j);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[j]),
                                                                        __builtin_bit_cast(bf16x8, fa[i]), acc[i][j], 0, 0, 0);
                if (h == 0) read_a(st, 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (h == 0) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) read_b(st, 1, j);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's copy has landed ...
        lds_barrier();                        // ... and everyone's; every read of stage st is done
    }

    // acc[i][j] holds C^T of tile (i, j): lane (m16, q4) element e is
    // C[row 16i + m16][column 16j + 4q4 + e]
    TC* Cp = static_cast<TC*>(a.C);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + wm + 16 * i + m16;
        if (row >= a.M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t col = n0 + wn + 16 * j + 4 * q4;
            TC* p = Cp + row * a.ldc + col;
            if (col + 3 < a.N) {
                if constexpr (sizeof(TC) == 4) {
                    *reinterpret_cast<f32x4*>(p) = acc[i][j];
                } else {
                    // float -> bfloat16 by the hardware conversion (round to nearest even)
                    const f32x4 v = acc[i][j];
                    typedef __bf16 b4_t __attribute__((ext_vector_type(4)));
                    *reinterpret_cast<b4_t*>(p) = b4_t{(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < a.N) st(p + e, acc[i][j][e]);
            }
        }
    }
}

// ------------------------------------------------------------ narrow kernel
// C[M, N <= 64] (the last N mod 256 columns of a wide product, such as the 64
// beta columns of the input projection): a 256 x 64 tile per workgroup leaves
// M / 256 workgroups, each walking all of K in latency-bound steps. Here a
// workgroup takes 32 rows and the four wavefronts split K four ways, each
// loading its operand fragments straight from memory into registers (a row's
// 128-byte line per 64-wide K step, the next step's fragments in flight during
// this step's products); the four partial tiles are summed through LDS.
constexpr int kNarrowRows = 32;

template <typename TC>
__global__ __launch_bounds__(256) void gemm_narrow_kernel(GemmArgs a)
{
    __shared__ f32x4 part[3][2][4][64];  // the partial tiles of wavefronts 1 .. 3
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * kNarrowRows;
    const int64_t rows_a = min<int64_t>(kNarrowRows, a.M - m0);
    const rsrc_t ra = make_rsrc(static_cast<const bf16_t*>(a.A) + m0 * a.lda, ((rows_a - 1) * a.lda + a.K) * 2);
    const rsrc_t rb = make_rsrc(a.B, ((a.N - 1) * a.ldb + a.K) * 2);
    const int kq = (int)(a.K / 4);                  // this wavefront's K range: [wave kq, (wave + 1) kq)
    const int nk = kq / 64;
    // lane (m16, q4): row 16 i + m16, K elements 8 q4 .. +7 of each 32-wide half
    int offa[2], offb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) offa[i] = (int)((16 * i + m16) * a.lda * 2) + (wave * kq + 8 * q4) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) offb[j] = (int)((16 * j + m16) * a.ldb * 2) + (wave * kq + 8 * q4) * 2;
    u32x4_t fa[2][2][2], fb[2][4][2];  // [buffer][tile][K half]
    auto load = [&](int kt, int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[buf][i][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, offa[i], (kt * 64 + 32 * h) * 2, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fb[buf][j][h] = __builtin_amdgcn_raw_buffer_load_b128(rb, offb[j], (kt * 64 + 32 * h) * 2, 0);
        }
    };
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    load(0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (kt + b >= nk) break;
            if (kt + b + 1 < nk) load(kt + b + 1, b ^ 1);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, fb[b][j][h]), __builtin_bit_cast(bf16x8, fa[b][i][h]), acc[i][j],
                            0, 0, 0);
        }
    }
    // acc[i][j] holds C^T of tile (i, j): lane (m16, q4) element e is
    // C[row 16i + m16][column 16j + 4q4 + e]; wavefronts 1 .. 3 hand theirs to 0
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) part[wave - 1][i][j][lane] = acc[i][j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += part[w][i][j][lane];
    TC* Cp = static_cast<TC*>(a.C);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t row = m0 + 16 * i + m16;
        if (row >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = 16 * j + 4 * q4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < a.N) st(Cp + row * a.ldc + col + e, acc[i][j][e]);
        }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s)
{
    // the main kernel's copies address rows through 32-bit offsets
    const bool main_path = a.K % 64 == 0 && (int64_t)TM * a.lda * 2 < ((int64_t)1 << 31) &&
                           (int64_t)TN * a.ldb * 2 < ((int64_t)1 << 31);
    if (main_path) {
        // whole 256-column tiles, then the last N mod 256 columns in 64- or
        // 128-column tiles (the 64 columns of the beta projection in the
        // 41,024-wide input projection: one more round of 32 workgroups)
        const int64_t tiles_m = (a.M + TM - 1) / TM;
        GemmArgs m = a;
        m.N = a.N / TN * TN;
        if (m.N > 0) {
            dim3 grid((unsigned)(tiles_m * (m.N / TN))), block(256);
            if (a.c_dtype == F32) hipLaunchKernelGGL((gemm256_kernel<float, 8>), grid, block, 0, s, m);
            else hipLaunchKernelGGL((gemm256_kernel<bf16_t, 8>), grid, block, 0, s, m);
        }
        GemmArgs r = a;
        r.N = a.N - m.N;
        if (r.N > 0 && r.N <= 64 && a.K % 256 == 0) {
            // up to 64 columns left: 32-row workgroups with K split four ways
            r.B = static_cast<const bf16_t*>(a.B) + m.N * a.ldb;
            r.C = static_cast<uint8_t*>(a.C) + m.N * (a.c_dtype == F32 ? 4 : 2);
            const dim3 grid((unsigned)((a.M + kNarrowRows - 1) / kNarrowRows)), block(256);
            if (a.c_dtype == F32) hipLaunchKernelGGL((gemm_narrow_kernel<float>), grid, block, 0, s, r);
            else hipLaunchKernelGGL((gemm_narrow_kernel<bf16_t>), grid, block, 0, s, r);
        } else if (r.N > 0) {
            r.B = static_cast<const bf16_t*>(a.B) + m.N * a.ldb;
            r.C = static_cast<uint8_t*>(a.C) + m.N * (a.c_dtype == F32 ? 4 : 2);
            const int nj = r.N <= 64 ? 2 : (r.N <= 128 ? 4 : 8);
            dim3 grid((unsigned)(tiles_m * ((r.N + 32 * nj - 1) / (32 * nj)))), block(256);
#define KDA_GEMM_REM(NJ)                                                                            \
    if (a.c_dtype == F32) hipLaunchKernelGGL((gemm256_kernel<float, NJ>), grid, block, 0, s, r);     \
    else hipLaunchKernelGGL((gemm256_kernel<bf16_t, NJ>), grid, block, 0, s, r);
            if (nj == 2) { KDA_GEMM_REM(2) }
            else if (nj == 4) { KDA_GEMM_REM(4) }
            else { KDA_GEMM_REM(8) }
#undef KDA_GEMM_REM
        }
        return hipGetLastError();
    }
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM)), block(kThreads);
    if (a.c_dtype == F32)
        hipLaunchKernelGGL(gemm_kernel<float>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gemm_kernel<bf16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
