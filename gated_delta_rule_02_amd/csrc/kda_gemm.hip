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
// accumulator registers: one wavefront per SIMD), K steps of 32 in four LDS
// stages filled by buffer-to-LDS copies that the wavefronts issue three steps
// ahead, and operand fragments read one step ahead. Per K step a wavefront
// reads 16 KiB of operands from LDS for 64 MFMAs, half the LDS rate the MFMAs
// could use. The stage
// layout is row major with the 16-byte K chunks of each row XOR-swizzled by
// (row / 4) mod 4, so that the 16 rows an MFMA operand read touches fall in
// distinct banks; the swizzle is applied by choosing each lane's global
// source address (a buffer-to-LDS copy writes lane l to byte 16 l of its
// 1 KiB destination). The products are formed transposed
// (B tile x A tile^T): each lane then holds four consecutive columns of one
// row of C, stored with one 16-byte (float32) or 8-byte (bfloat16) access.
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
constexpr int TM = 256, TN = 256, TK = 32;   // workgroup tile and K step
constexpr int kStages = 4;                   // K steps in LDS: the copies run 3 steps ahead
constexpr int kStageBytes = TM * TK * 2;      // one operand's stage: 256 rows x 64 B
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte offset of 16-byte chunk c (0..3) of row r of a stage: the chunks
// are XOR-swizzled by (r / 4) mod 4, so the 16 rows of an operand read cover
// all 64 banks
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// NJ: 16-column MFMA tiles per wavefront in N (8: the 256 x 256 tile; 2 or 4:
// a 256 x 64 or 256 x 128 tile for the last N mod 256 columns, so that they
// cost a fraction of a full tile instead of a whole one)
template <typename TC, int NJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm256_kernel(GemmArgs a)
{
    constexpr int TNW = 32 * NJ;         // columns of C per workgroup
    constexpr int kBCopy = TNW / 64;     // B copy instructions per wavefront and K step
    constexpr int kCopyInstr = 4 + kBCopy;
    constexpr int kWaitOneCopy = 0x0f70 | kCopyInstr;  // s_waitcnt vmcnt(kCopyInstr)
    static_assert(NJ == 2 || NJ == 4 || NJ == 8, "64, 128 or 256 columns");
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages][2][kStageBytes];  // [stage][A, B]
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

    // copy of K step kt into stage st: 16 instructions for A (4 per
    // wavefront) and TNW / 16 for B (kBCopy per wavefront); instruction i
    // covers rows 16i .. 16i+15, lane l row 16i + l/4 and LDS chunk slot l%4,
    // which holds K chunk slot ^ ((row/4) mod 4)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)&smem[0][0][0];
    const int lrow = lane >> 2, lslot = lane & 3;
    auto copy_part = [&](int kt, int st, int j) {
        const int i = wave * 4 + j;
        const int row = 16 * i + lrow;
        const int chunk = lslot ^ ((row >> 2) & 3);
        const int koff = (kt * TK + chunk * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(uintptr_t)(lds0 + (st * 2 + 0) * kStageBytes + i * 1024),
                                                 16, (int)(row * a.lda * 2) + koff, 0, 0, 0);
        if (j < kBCopy) {
            // B has TNW rows: instruction ib = wave * kBCopy + j covers rows 16 ib .. 16 ib + 15
            const int ib = wave * kBCopy + j;
            const int rowb = 16 * ib + lrow;
            const int chunkb = lslot ^ ((rowb >> 2) & 3);
            const int koffb = (kt * TK + chunkb * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(uintptr_t)(lds0 + (st * 2 + 1) * kStageBytes + ib * 1024),
                                                     16, (int)(rowb * a.ldb * 2) + koffb, 0, 0, 0);
        }
    };
    auto copy = [&](int kt, int st) {
#pragma unroll
        for (int j = 0; j < 4; ++j) copy_part(kt, st, j);
    };

    f32x4 acc[8][NJ];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Pipeline: step kt computes on stage kt % 4 with operand fragments read
    // during step kt - 1. Between its MFMAs it issues the copy of step kt + 3
    // (each copy instruction waits for the compute unit's address unit, 1 KiB
    // at 64 B per clock shared by the four wavefronts, which the matrix unit's
    // work hides; issued up front they delayed every step's MFMAs) and reloads
    // each A fragment for step kt + 1 as soon as its last MFMA is issued (the
    // B fragments, used by every row, after the last row). At its end it waits
    // for the copy of step kt + 2, so that after the barrier stage kt + 2 is
    // complete for the next step's early reads. The compiler does not track
    // the copies: the waits are explicit. A copy is kCopyInstr instructions
    // per wavefront (4 of A, kBCopy of B) and copies complete in order, so
    // "copy c has landed" is vmcnt(kCopyInstr x the copies issued after it).
    const int nk = (int)(a.K / TK);
    u32x4_t fa[8], fb[NJ];
    auto read_a = [&](int kt, int i) {
        fa[i] = *reinterpret_cast<const u32x4_t*>(&smem[kt % kStages][0][0] + swz(wm + 16 * i + m16, q4));
    };
    auto read_b = [&](int kt, int j) {
        fb[j] = *reinterpret_cast<const u32x4_t*>(&smem[kt % kStages][1][0] + swz(wn + 16 * j + m16, q4));
    };
    for (int p = 0; p < kStages - 1 && p < nk; ++p) copy(p, p);
    if (nk > 2) __builtin_amdgcn_s_waitcnt(kWaitOneCopy);  // steps 0 and 1 landed (step 2 in flight)
    else __builtin_amdgcn_s_waitcnt(0x0f70);               // vmcnt(0)
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) read_a(0, i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) read_b(0, j);
    for (int kt = 0; kt < nk; ++kt) {
        const bool cp = kt + kStages - 1 < nk, nx = kt + 1 < nk;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[j]),
                                                                    __builtin_bit_cast(bf16x8, fa[i]), acc[i][j], 0, 0, 0);
            if (i < 4 && cp) copy_part(kt + kStages - 1, (kt + kStages - 1) % kStages, i);
            if (nx) read_a(kt + 1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (nx) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) read_b(kt + 1, j);
        }
        // the copy of step kt + 2 has landed (this wavefront's part) ...
        if (cp) __builtin_amdgcn_s_waitcnt(kWaitOneCopy);  // vmcnt(kCopyInstr)
        else __builtin_amdgcn_s_waitcnt(0x0f70);           // vmcnt(0)
        lds_barrier();  // ... and everyone's; every read of stage kt % 4 is done
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
        if (r.N > 0) {
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
