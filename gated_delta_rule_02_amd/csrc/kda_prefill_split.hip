// kda_prefill_split.hip -- two-pass chunked KDA prefill (bfloat16 inputs).
//
// The single-pass kernel runs the whole chain of a (sequence, head) on one
// compute unit, so a single long sequence with 64 heads occupies a quarter of
// the GPU and every chunk pays the latency of its chunk-local phases. Here the
// chunk-local work, which does not depend on the state, runs for all chunks at
// once, and only the state recurrence stays sequential:
//
//   intra pass  (workgroup per (sequence, head, group of chunks); P0 .. P2b of
//               kda_chunk.h, then a block forward substitution) writes, per
//               chunk, in the operand layouts of the state pass:
//                 -W = -(I + A)^-1 diag(beta) (K o 2^B)       tokens x dk
//                 U' =  (I + A)^-1 diag(beta) V               tokens x dv
//                 Q~ =  Q o 2^B                               tokens x dk
//                 Kbar^T = (K o 2^(b_C - B))^T                dk x tokens
//                 P (lower triangle incl. the diagonal)        tokens x tokens
//                 2^b_C                                        dk
//   state pass  (workgroup per (sequence, head, 32 value columns); the chunks
//               of the sequence in order), from the identities of the chunk
//               form in kda_chunk.h with U = U' + (-W) S0:
//                 U   = U' + (-W) S
//                 O   = scale (Q~ S + P U)
//                 S  <- Diag(2^b_C) S + Kbar^T U
//               four 64 x 128 x 16 or 128 x 64 x 16 MFMA products per chunk and
//               wavefront, with no triangular solve left on the chain.
//
// The products are stored as float16 (their magnitudes are bounded by the
// key, value and state magnitudes; entries that underflow are below 2^-24 of
// the terms they multiply), which keeps the workspace at 70.5 KiB per chunk
// and head. Chunks are processed in windows of up to `nwin` chunks per
// sequence so that the workspace is bounded; between windows the state pass
// carries the state through a float32 buffer in the workspace.
#include <algorithm>
#include <mutex>

#include "kda_chunk.h"

namespace kda {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Byte offsets inside one chunk slot. A-operand layout [t][s][lane][8 halves]:
// for the 16-row tile t and the 32-wide K step s, lane (m = lane % 16,
// qq = lane / 16) holds X[16t + m][32s + 4qq .. +3] followed by
// X[16t + m][32s + 16 + 4qq .. +3].
constexpr int kNegW = 0;        // -W       [4][4][64][8] f16
constexpr int kQt = 16384;      // Q~       [4][4][64][8] f16
constexpr int kKbT = 32768;     // Kbar^T   [8][2][64][8] f16
constexpr int kPm = 49152;      // P        [6][64][8] f16: the fragments (t, s) with 2s <= t, in the order
                                // (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); the two above the diagonal are zero
constexpr int kDma = 55296;     // the four matrices above: copied to LDS as one block
constexpr int kUp = 55296;      // U' in the accumulator layout [8 j][4 t][64][4] f16:
                                // lane (n, q) of column tile j holds U'[16t + 4q + i][16j + n]
constexpr int kDc = 71680;      // 2^b_C    [128] f32
constexpr int kSlot = 72192;
constexpr int kStateWaves = 2;  // compute wavefronts of the state pass
constexpr int kStateThreads = 64 * (kStateWaves + 1);  // + a loader wavefront
constexpr int kStUp = kDma;     // offset of U' (2 KiB per 16-column tile) in an LDS stage
// LDS stage of a state-pass workgroup with `tiles` 16-column tiles: operand
// block, U' of its tiles, 2^b_C (copied as 1 KiB: the tail is padding)
__host__ __device__ constexpr int state_stage_bytes(int tiles) { return kDma + tiles * 2048 + 1024; }

struct SplitArgs {
    PrefillArgs p;
    uint8_t* ws;      // slots [num_seqs][H][nwin]
    float* carry;     // [num_seqs][H][128][128] between windows, or null
    int64_t chunk0;   // first chunk (of each sequence) in this window
    int nwin;         // chunk slots per (sequence, head)
    int groups;       // intra-pass workgroups per (sequence, head)
    int map_half;     // segment maps: state-pass workgroups of each half of the grid
};

__device__ __forceinline__ void seq_bounds(const PrefillArgs& a, int n, int64_t& s, int64_t& e)
{
    if (a.cu_seqlens) {
        s = a.cu_seqlens[n];
        e = a.cu_seqlens[n + 1];
    } else {
        s = (int64_t)n * a.seq_len;
        e = s + a.seq_len;
    }
}

// ------------------------------------------------------------- intra pass
// Block column I of T = (I + A)^-1 below the diagonal (A strictly lower and
// beta-scaled, stored negated in An; T_RR in Tb): T_RI = T_RR sum_{I<=J<R}
// (-A_RJ) T_JI for R = I+1 .. 3, each block rounded to float16 once. The
// running blocks T_JI stay in registers in the B-operand layout (= the
// accumulator layout of the product that made them); Tm receives them row
// major, the A-operand layout of the products with T.
template <int I, typename SM>
__device__ __forceinline__ void inverse_column(SM& sm, _Float16 (*Tm)[16][BLD], int m16, int q4)
{
    using O = Ops<false>;
    using F4 = typename O::F4;
    constexpr int NB = SM::NB;
    F4 tc[NB];
#pragma unroll
    for (int i = 0; i < 4; ++i) tc[I][i] = sm.Tb[I][4 * q4 + i][m16];  // T_II in the B layout
#pragma unroll
    for (int R = I + 1; R < NB; ++R) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = I; J < R; ++J) acc = O::mma16(O::lds(&sm.An[pair_id(R, J)][m16][4 * q4]), tc[J], acc);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        tc[R] = O::cvt(O::mma16(O::lds(&sm.Tb[R][m16][4 * q4]), O::cvt(acc), z));
#pragma unroll
        for (int i = 0; i < 4; ++i) Tm[pair_id(R, I)][4 * q4 + i][m16] = tc[R][i];
    }
}

// POL: cache policy of the input loads (0 or kStream); NOQ: segment maps
// (no query side: Q~ and P are neither formed nor stored); GATE: g and beta
// formed from the projection rows (the gate prologue inside the prefill)
template <typename TIN, int POL, bool NOQ = false, bool GATE = false>
__global__ __launch_bounds__(kThreads) void intra_kernel(SplitArgs sa)
{
    using O = Ops<false>;
    using OT = _Float16;
    using F4 = typename O::F4;
    using F8 = typename O::F8;
    using SM = Smem<false>;
    constexpr int C = SM::C;
    constexpr int NB = SM::NB;
    static_assert(C == 64 && NB == 4, "slot layout assumes 64-token chunks");

    __shared__ SM sm;
    __shared__ __attribute__((aligned(16))) _Float16 Tm[SM::NPAIR][16][BLD];  // T = (I + A)^-1 below the diagonal
    const PrefillArgs& a = sa.p;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int m16 = lane & 15;
    const int q4 = lane >> 4;

    const int grp = blockIdx.x % sa.groups;
    const int u = blockIdx.x / sa.groups;  // n * H + h
    const int h = u % a.H;
    const int n = u / a.H;
    int64_t seq_s, seq_e;
    seq_bounds(a, n, seq_s, seq_e);
    const int64_t nchunks = (seq_e - seq_s + C - 1) / C;
    const int64_t c_end = min<int64_t>(nchunks, sa.chunk0 + sa.nwin);
    const int64_t c_first = sa.chunk0 + grp;
    if (c_first >= c_end) return;

    const TIN* vg = static_cast<const TIN*>(a.v);
    uint8_t* slots = sa.ws + (size_t)u * sa.nwin * kSlot;

    Front<false, TIN, 2, true, POL, NOQ, GATE> fr(sm, a, h);
    {
        const int64_t cs = seq_s + c_first * C;
        fr.load(cs, (int)min<int64_t>(C, seq_e - cs), vg);
    }

    for (int64_t c = c_first; c < c_end; c += sa.groups) {
        const int64_t cs = seq_s + c * C;
        const int64_t cn = c + sa.groups;  // this workgroup's next chunk
        const int64_t csn = seq_s + cn * C;
        const bool more = cn < c_end;

        fr.p0();
        __syncthreads();
        fr.p1();
        // the next chunk's inputs, issued in three parts (g, k, beta; q; v) so
        // that they stream in behind P2, P2c and the products rather than
        // stalling one phase
        const int ntn = (int)min<int64_t>(C, seq_e - csn);
        if (more) fr.template load<1>(csn, ntn, vg);
        __syncthreads();
        fr.p2();
        if (more) fr.template load<2>(csn, ntn, vg);
        __syncthreads();
        fr.p2b();
        // ---- P2c: the blocks of T = (I + A)^-1 below the diagonal, one block
        // column per wavefront: T_RI = T_RR sum_{I<=J<R} (-A_RJ) T_JI
        if (wave == 0) inverse_column<0>(sm, Tm, m16, q4);
        else if (wave == 1) inverse_column<1>(sm, Tm, m16, q4);
        else if (wave == 2) inverse_column<2>(sm, Tm, m16, q4);
        if (more) fr.template load<4>(csn, ntn, vg);
        __syncthreads();

        // ---- -W and U' as products with T: Z_R = sum_{I<=R} T_RI X_I
        // (independent block rows). The right-hand sides come transposed from
        // P2b, so that a lane reads the four tokens of its channel that it
        // holds as an operand at once. U' is formed as T X (its accumulator
        // layout is the slot's), -W as (T X)^T = X^T T^T: the same registers
        // with the operands swapped, which leaves four consecutive channels of
        // one token per lane, stored straight to the slot.
        uint8_t* slot = slots + (size_t)(c - sa.chunk0) * kSlot;
        // wavefront 2p forms -W for the tiles 2p, 2p + 1 (so that each lane
        // holds the whole 16-byte slot fragment: channels 32p + 4q4 .. +3 and
        // 32p + 16 + 4q4 .. +3 of one token), wavefront 2p + 1 forms U' for
        // the same two tiles
        const bool isW = !(wave & 1);
        const int col0 = 32 * (wave >> 1) + m16;  // this lane's column of the first tile
        const OT(*X)[SM::LDT] = isW ? sm.key.x.XWt : sm.key.x.XUt;
        F4 X0[NB], X1[NB];
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            X0[I] = O::lds(&X[col0][16 * I + 4 * q4]);
            X1[I] = O::lds(&X[col0 + 16][16 * I + 4 * q4]);
        }
        // block (R, I) of T in the A-operand layout
        auto tblk = [&](int Rr, int I) {
            return I == Rr ? O::lds(&sm.Tb[Rr][m16][4 * q4]) : O::lds(&Tm[pair_id(Rr, I)][m16][4 * q4]);
        };
#pragma unroll
        for (int Rr = 0; Rr < NB; ++Rr) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
            if (isW) {
#pragma unroll
                for (int I = 0; I + 1 <= Rr; I += 2) {
                    const F8 t2 = O::cat2(tblk(Rr, I), tblk(Rr, I + 1));
                    a0 = O::mma32(O::cat2(X0[I], X0[I + 1]), t2, a0);
                    a1 = O::mma32(O::cat2(X1[I], X1[I + 1]), t2, a1);
                }
                if (!(Rr & 1)) {
                    const F4 tb = tblk(Rr, Rr);
                    a0 = O::mma16(X0[Rr], tb, a0);
                    a1 = O::mma16(X1[Rr], tb, a1);
                }
                // lane (token m16, q4) holds the fragment (tile Rr, K step p) of lane m16 + 16 q4
                *reinterpret_cast<F8*>(slot + kNegW + ((Rr * 4 + (wave >> 1)) * 64 + lane) * 16) =
                    O::cat2(O::cvt(a0), O::cvt(a1));
            } else {
#pragma unroll
                for (int I = 0; I + 1 <= Rr; I += 2) {
                    const F8 t2 = O::cat2(tblk(Rr, I), tblk(Rr, I + 1));
                    a0 = O::mma32(t2, O::cat2(X0[I], X0[I + 1]), a0);
                    a1 = O::mma32(t2, O::cat2(X1[I], X1[I + 1]), a1);
                }
                if (!(Rr & 1)) {
                    const F4 tb = tblk(Rr, Rr);
                    a0 = O::mma16(tb, X0[Rr], a0);
                    a1 = O::mma16(tb, X1[Rr], a1);
                }
                // U' in its accumulator layout, tiles 2p and 2p + 1
                *reinterpret_cast<F4*>(slot + kUp + (((wave - 1) * 4 + Rr) * 64 + lane) * 8) = O::cvt(a0);
                *reinterpret_cast<F4*>(slot + kUp + ((wave * 4 + Rr) * 64 + lane) * 8) = O::cvt(a1);
            }
        }
        // (no barrier: the products wrote nothing to LDS, and what the copy
        // reads was complete before the last one)

        // ---- the operand matrices in the A-operand layout, 16 bytes per lane
        // (every LDS read is issued before the first store, so that they are
        // in flight together)
        h8 cq[2] = {}, ck[2], cp = {};
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            if constexpr (NOQ) break;
            const int idx = tid + kThreads * k2;  // [t 4][s 4][lane 64]
            const int t = idx >> 8, s = (idx >> 6) & 3, l = idx & 63;
            const int row = 16 * t + (l & 15), col = 32 * s + 4 * (l >> 4);
            cq[k2] = cat(*reinterpret_cast<const h4*>(&sm.key.x.Qt[row][col]),
                         *reinterpret_cast<const h4*>(&sm.key.x.Qt[row][col + 16]));
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int idx = tid + kThreads * k2;  // [t 8][s 2][lane 64]
            const int t = idx >> 7, s = (idx >> 6) & 1, l = idx & 63;
            const int row = 16 * t + (l & 15), col = 32 * s + 4 * (l >> 4);
            ck[k2] = cat(*reinterpret_cast<const h4*>(&sm.KbT[row][col]),
                         *reinterpret_cast<const h4*>(&sm.KbT[row][col + 16]));
        }
        if (!NOQ && tid < 6 * 64) {
            const int i = tid >> 6, l = tid & 63;  // fragment i = (t, s) with 2s <= t
            const int t = i < 2 ? i : 2 + (i - 2) / 2, s = i < 2 ? 0 : (i - 2) % 2;
            const int m = l & 15, cq4 = 4 * (l >> 4);
            const h4 zero = {(OT)0.f, (OT)0.f, (OT)0.f, (OT)0.f};
            const h4 lo = *reinterpret_cast<const h4*>(&sm.Pb[tri_id(t, 2 * s)][m][cq4]);
            const h4 hi = (2 * s + 1 <= t) ? *reinterpret_cast<const h4*>(&sm.Pb[tri_id(t, 2 * s + 1)][m][cq4]) : zero;
            cp = cat(lo, hi);
        }
        f32x4 cdc = {0.f, 0.f, 0.f, 0.f};
        if (tid < D / 4) cdc = ld4f(&sm.bC[4 * tid]);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int idx = tid + kThreads * k2;
            if constexpr (!NOQ) *reinterpret_cast<h8*>(slot + kQt + idx * 16) = cq[k2];
            *reinterpret_cast<h8*>(slot + kKbT + idx * 16) = ck[k2];
        }
        if (!NOQ && tid < 6 * 64) *reinterpret_cast<h8*>(slot + kPm + tid * 16) = cp;
        if (tid < D / 4) *reinterpret_cast<f32x4*>(slot + kDc + tid * 16) = cdc;
        // the next P0 writes only Gp and beta, which nothing above reads; its
        // barrier orders these LDS reads before P1 reuses the region

    }
}

// ------------------------------------------------------------- state pass
// The form for 64-column workgroups and segment maps (32-column workgroups
// of an ordinary prefill take the role-split form below). Three wavefronts:
// two compute wavefronts (one or two 16-column tiles of the state each) and a
// loader that copies each chunk's operands into an LDS stage with
// buffer-to-LDS loads (two stages, one chunk ahead). Each role waits only on
// its own memory counter; one barrier per chunk hands a stage from the loader
// to the compute wavefronts. (A fourth wavefront that touched the chunks two
// to four ahead, to pull them into L2 early, made the pass slower: its reads
// competed with the loader's, and lines it fetched were evicted before use,
// so the pass fetched 1.65x the workspace instead of 1.04x.)
//
// The output is formed transposed, O^T = S^T Q~^T + U^T P^T: the 16 x 16 x 32
// MFMA takes the same lane layout for its two operands, so the registers that
// hold S (or U) as a B operand serve as the A operand of the transposed
// product, and the stored A-operand layouts of Q~ and P serve as B operands.
// The result then holds four consecutive output columns of one token per lane
// (16-byte stores) instead of four tokens of one column.
// POL: cache policy of the output stores (0 or kStream); MAP: segment maps
template <typename TOUT, int TPW, int POL, bool MAP>
__global__ __launch_bounds__(kStateThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void state_kernel(SplitArgs sa)
{
    constexpr int kTiles = kStateWaves * TPW;      // 16-column tiles per workgroup
    constexpr int kColGroups = D / (16 * kTiles);  // workgroups per (sequence, head)
    constexpr int kStage = state_stage_bytes(kTiles);
    constexpr int kStDc = kStUp + kTiles * 2048;   // offset of 2^b_C in a stage
    __shared__ __attribute__((aligned(16))) uint8_t buf[2][kStage];
    const PrefillArgs& a = sa.p;
    constexpr int C = 64;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int m16 = lane & 15;
    const int q4 = lane >> 4;
    const bool compute = wave < kStateWaves;
    const bool loader = wave == kStateWaves;

    // Workgroup ids are dealt to the 8 XCDs round robin; the kColGroups
    // workgroups of one (sequence, head) get ids congruent mod 8, so they read
    // the chunk products through the same L2.
    // Segment maps: the grid is doubled; its first half carries M (from the
    // identity, with U' = 0: the map's linear part), the second half N (from
    // zero); no output is formed.
    constexpr bool map = MAP;
    const int half = map ? (int)(blockIdx.x / sa.map_half) : 1;  // 0: M, 1: N (or the ordinary state)
    const int bid = map ? (int)(blockIdx.x % sa.map_half) : (int)blockIdx.x;
    const int jq = (bid >> 3) % kColGroups;
    const int u = (bid & 7) + 8 * ((bid >> 3) / kColGroups);  // n * H + h
    if (u >= a.num_seqs * a.H) return;
    const int h = u % a.H;
    const int n = u / a.H;
    int64_t seq_s, seq_e;
    seq_bounds(a, n, seq_s, seq_e);
    const int64_t nchunks = (seq_e - seq_s + C - 1) / C;
    const int64_t c_end = min<int64_t>(nchunks, sa.chunk0 + sa.nwin);
    const int nch = (int)max<int64_t>(0, c_end - sa.chunk0);
    const int jl = compute ? wave * TPW : 0;  // this wavefront's first tile within the workgroup
    const int j0 = kTiles * jq + jl;         // its first 16-column tile; tile p is j0 + p
    const size_t sbase = (size_t)u * D * D;

    // M's half starts from the identity and N's from zero; across windows each
    // is carried in its own output (every workgroup reads and writes only its
    // own columns)
    float* const mapout = half ? a.sT : a.map_M;
    if (nch == 0) {
        // an empty sequence still has a final state: the initial one (for a
        // segment map: M = I, N = 0)
        if (compute && sa.chunk0 == 0 && (map || a.sT)) {
            float* const dst = map ? mapout : a.sT;
#pragma unroll
            for (int p = 0; p < TPW; ++p) {
                int off = 4 * q4 * D + 16 * (j0 + p) + m16;
                asm volatile("" : "+v"(off));
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const size_t e = sbase + off + (size_t)(16 * t + i) * D;
                        dst[e] = map ? ((half == 0 && 16 * t + 4 * q4 + i == 16 * (j0 + p) + m16) ? 1.0f : 0.0f)
                                     : (a.s0 ? a.s0[e] : 0.0f);
                    }
            }
        }
        return;
    }
    const float* sin = map ? (sa.chunk0 == 0 ? nullptr : mapout) : (sa.chunk0 == 0 ? a.s0 : sa.carry);
    float* sout = map ? mapout : (c_end >= nchunks ? a.sT : sa.carry);
    const bool ident = map && half == 0 && sa.chunk0 == 0;  // M's first window starts from I
    const bool zeroU = map && half == 0;                      // M's half: U' = 0

    // this (sequence, head)'s slots through one descriptor; the wave-uniform
    // parts of every address are scalar
    const uint8_t* slots = sa.ws + (size_t)u * sa.nwin * kSlot;
    const rsrc_t rs = make_rsrc(slots, (int64_t)nch * kSlot);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)&buf[0][0];
    // loader: chunk c into stage b, 1 KiB per instruction (lane l moves bytes
    // 16 l .. 16 l + 15): the operand block, then U' of this workgroup's
    // tiles, then 2^b_C (the instruction moves 1 KiB; the tail is padding).
    // Measured alternatives moved the same ~61 KiB per chunk and compute unit
    // no faster: two loader wavefronts, or loads through registers + LDS stores.
    auto dma = [&](int c, int b) {
        const uint32_t st = lds0 + b * kStage;
#pragma unroll
        for (int i = 0; i < kDma / 1024; ++i) {
            // segment maps read neither Q~ nor P
            if (MAP && ((i >= kQt / 1024 && i < kKbT / 1024) || i >= kPm / 1024)) continue;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + i * 1024), 16, lane * 16,
                                                     c * kSlot + i * 1024, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * kTiles; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + kStUp + i * 1024), 16, lane * 16,
                                                     c * kSlot + kUp + jq * kTiles * 2048 + i * 1024, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + kStDc), 16, lane * 16,
                                                 c * kSlot + kDc, 0, 0);
    };

    f32x4 S[TPW][8];  // S[p][t][i] = S[16t + 4q + i][16 (j0 + p) + m16]
    if (compute) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            if (sin) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[p][t][i] = sin[sbase + (size_t)(16 * t + 4 * q4 + i) * D + 16 * (j0 + p) + m16];
            } else if (ident) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[p][t][i] = (16 * t + 4 * q4 + i == 16 * (j0 + p) + m16) ? 1.0f : 0.0f;
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) S[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    if (loader) {
        dma(0, 0);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }

    const int ts = a.H * D;
    TOUT* og = static_cast<TOUT*>(a.o);
    // snapshots: chunks left to the next multiple of the interval, and its index
    const int snap_ic = a.snap ? (int)(a.snap_interval / C) : 1;
    int snap_left = snap_ic - (int)(sa.chunk0 % snap_ic);
    int snap_j = (int)(sa.chunk0 / snap_ic);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // stage c & 1 holds chunk c
        if (loader) {
            if (c + 1 < nch) dma(c + 1, (c + 1) & 1);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the stage is complete before the next barrier
            continue;
        }
        const uint8_t* st = &buf[c & 1][0];
        const h8* nw = reinterpret_cast<const h8*>(st + kNegW);
        const h8* qt = reinterpret_cast<const h8*>(st + kQt);
        const h8* kb = reinterpret_cast<const h8*>(st + kKbT);
        const h8* pm = reinterpret_cast<const h8*>(st + kPm);

        // The operand reads run one group ahead of the MFMAs that consume them
        // (LDS latency is otherwise exposed on every product); each operand
        // read serves the wavefront's TPW tiles.
        h8 sb[TPW][4];  // S as the B operand (and S^T as the A operand) of a K step over dk
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[p][s] = cat(to_h4(S[p][2 * s]), to_h4(S[p][2 * s + 1]));
        f32x4 U[TPW][4], Ot[TPW][4];  // U[p][t]: tokens 16t.. x tile p; Ot[p][t]: tile p x tokens 16t..
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const h4 up = *reinterpret_cast<const h4*>(st + kStUp + (((jl + p) * 4 + t) * 64 + lane) * 8);
                U[p][t] = zeroU ? f32x4{0.f, 0.f, 0.f, 0.f} : f32x4{(float)up[0], (float)up[1], (float)up[2], (float)up[3]};
                Ot[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        h8 an[2][4], aq[2][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            an[0][t] = nw[(t * 4 + 0) * 64 + lane];
            if constexpr (!MAP) aq[0][t] = qt[(t * 4 + 0) * 64 + lane];
        }
        h8 ap[6], ak[16];  // P and Kbar^T operands, read during the first products
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cur = s & 1, nxt = cur ^ 1;
            if (s < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    an[nxt][t] = nw[(t * 4 + s + 1) * 64 + lane];
                    if constexpr (!MAP) aq[nxt][t] = qt[(t * 4 + s + 1) * 64 + lane];
                }
            } else if constexpr (!MAP) {
#pragma unroll
                for (int i = 0; i < 6; ++i) ap[i] = pm[i * 64 + lane];  // (t, s) with 2s <= t
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int p = 0; p < TPW; ++p) {
                    U[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(an[cur][t], sb[p][s], U[p][t], 0, 0, 0);
                    if constexpr (!MAP)
                        Ot[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sb[p][s], aq[cur][t], Ot[p][t], 0, 0, 0);
                }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ak[i] = kb[i * 64 + lane];  // [t][s] = index t * 2 + s
        h8 ub[TPW][2];  // U as the B operand (U^T as the A operand) of a K step over tokens
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
            for (int s = 0; s < 2; ++s) ub[p][s] = cat(to_h4(U[p][2 * s]), to_h4(U[p][2 * s + 1]));
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            if constexpr (MAP) break;  // segment maps form no output
            const int t = i < 2 ? i : 2 + (i - 2) / 2, s2 = i < 2 ? 0 : (i - 2) % 2;
#pragma unroll
            for (int p = 0; p < TPW; ++p)
                Ot[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ub[p][s2], ap[i], Ot[p][t], 0, 0, 0);
        }
        // state: S <- Diag(2^b_C) S + Kbar^T U
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 dc = *reinterpret_cast<const f32x4*>(st + kStDc + (16 * t + 4 * q4) * 4);
#pragma unroll
            for (int p = 0; p < TPW; ++p) {
                f32x4 acc = S[p][t] * dc;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[t * 2 + s], ub[p][s], acc, 0, 0, 0);
                S[p][t] = acc;
            }
        }
        // outputs: lane (token m16 of tile t, q4) holds columns 16j + 4 q4 .. +3;
        // rows past the sequence are dropped by the descriptor range
        const int64_t cs = seq_s + (sa.chunk0 + c) * C;
        const int ntok = (int)min<int64_t>(C, seq_e - cs);
        if constexpr (MAP) continue;  // segment maps: no output, no snapshots
        // state snapshot when a whole chunk ends on a multiple of the interval
        if (a.snap && --snap_left == 0) {
            if (ntok == C) {
#pragma unroll
                for (int p = 0; p < TPW; ++p)
                    store_state_slice(a.snap + (((size_t)n * a.snap_slots + snap_j) * a.H + h) * D * D, S[p], q4,
                                      16 * (j0 + p) + m16);
            }
            snap_left = snap_ic;
            ++snap_j;
        }
        const rsrc_t ro_ = make_rsrc(og + cs * ts, (int64_t)ntok * ts * (int64_t)sizeof(TOUT));
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            const int voff = (m16 * ts + h * D + 16 * (j0 + p) + 4 * q4) * (int)sizeof(TOUT);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 v = a.scale * Ot[p][t];
                if constexpr (sizeof(TOUT) == 4) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ro_, voff, 16 * t * ts * 4,
                                                           POL);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, to_b4(v)), ro_, voff,
                                                          16 * t * ts * 2, POL);
                }
            }
        }
    }
    if (!compute) {
        // no load may still be writing LDS when the workgroup ends
        __builtin_amdgcn_s_waitcnt(0x0f70);
        return;
    }
    if (sout) {
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
            int off = 4 * q4 * D + 16 * (j0 + p) + m16;
            asm volatile("" : "+v"(off));
            float* so = sout + sbase + off;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) so[(16 * t + i) * D] = S[p][t][i];
        }
    }
}

// ------------------------------------------------------- role-split state pass
// The same recurrence with the work of each 16-column tile shared by two
// compute wavefronts that run side by side on their own SIMDs:
//   A (the chain): U = U' + (-W) S, then S <- Diag(2^b_C) S + Kbar^T U;
//   B (the output): O^T = S^T Q~^T + U^T P^T and its stores.
// A hands S (for the next chunk) and U (after its first product) to B through
// LDS, as float16 B operands, double-buffered by chunk parity. The chain of a
// chunk is then two products of 16 MFMAs instead of all four products in one
// wavefront; with one wavefront per tile the pass was bound by that
// wavefront's chain, not by its loads. One barrier per chunk (the stage holds
// the chunk; S is published); U's hand-over is a per-tile LDS counter that B
// polls, so that the loader, which spends most of a chunk issuing the next
// one's copies, is not waited for in the middle of the chunk. Waves: 0 B,
// 1 A of tile 0; 2 B, 3 A of tile 1; 4 loader (on SIMD 0 with the lighter B
// wavefront).
constexpr int kRoleTiles = 2;                       // 16-column tiles per workgroup
constexpr int kRoleThreads = 64 * (2 * kRoleTiles + 1);
constexpr int kRoleStage = state_stage_bytes(kRoleTiles);

template <typename TOUT, int POL>
__global__ __launch_bounds__(kRoleThreads) void state_roles_kernel(SplitArgs sa)
{
    constexpr int kColGroups = D / (16 * kRoleTiles);  // workgroups per (sequence, head)
    constexpr int kStDc = kStUp + kRoleTiles * 2048;    // offset of 2^b_C in a stage
    __shared__ __attribute__((aligned(16))) uint8_t buf[2][kRoleStage];
    __shared__ h8 sbx[2][kRoleTiles][4][64];  // S before chunk c in [c & 1], B-operand layout
    __shared__ h8 ubx[2][kRoleTiles][2][64];  // U of chunk c in [c & 1], B-operand layout
    __shared__ int uflag[kRoleTiles];         // chunks whose U wavefront A has published
    const PrefillArgs& a = sa.p;
    constexpr int C = 64;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int m16 = lane & 15;
    const int q4 = lane >> 4;
    const bool loader = wave == 2 * kRoleTiles;
    const bool roleA = !loader && (wave & 1);
    const bool roleB = !loader && !(wave & 1);
    const int p = loader ? 0 : wave >> 1;  // this wavefront's tile within the workgroup

    // workgroups of one (sequence, head) get ids congruent mod 8 (one XCD)
    const int bid = (int)blockIdx.x;
    const int jq = (bid >> 3) % kColGroups;
    const int u = (bid & 7) + 8 * ((bid >> 3) / kColGroups);  // n * H + h
    if (u >= a.num_seqs * a.H) return;
    const int h = u % a.H;
    const int n = u / a.H;
    int64_t seq_s, seq_e;
    seq_bounds(a, n, seq_s, seq_e);
    const int64_t nchunks = (seq_e - seq_s + C - 1) / C;
    const int64_t c_end = min<int64_t>(nchunks, sa.chunk0 + sa.nwin);
    const int nch = (int)max<int64_t>(0, c_end - sa.chunk0);
    const int j = kRoleTiles * jq + p;  // this wavefront's 16-column tile
    const size_t sbase = (size_t)u * D * D;

    if (nch == 0) {
        // an empty sequence still has a final state: the initial one
        if (roleA && sa.chunk0 == 0 && a.sT) {
            int off = 4 * q4 * D + 16 * j + m16;
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t e = sbase + off + (size_t)(16 * t + i) * D;
                    a.sT[e] = a.s0 ? a.s0[e] : 0.0f;
                }
        }
        return;
    }
    const float* sin = sa.chunk0 == 0 ? a.s0 : sa.carry;
    float* sout = c_end >= nchunks ? a.sT : sa.carry;

    const uint8_t* slots = sa.ws + (size_t)u * sa.nwin * kSlot;
    const rsrc_t rs = make_rsrc(slots, (int64_t)nch * kSlot);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)&buf[0][0];
    // loader: chunk c into stage b, 1 KiB per instruction: the operand block,
    // U' of this workgroup's tiles, 2^b_C (the tail of its KiB is padding)
    auto dma = [&](int c, int b) {
        const uint32_t st = lds0 + b * kRoleStage;
#pragma unroll
        for (int i = 0; i < kDma / 1024; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + i * 1024), 16, lane * 16,
                                                     c * kSlot + i * 1024, 0, 0);
#pragma unroll
        for (int i = 0; i < 2 * kRoleTiles; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + kStUp + i * 1024), 16, lane * 16,
                                                     c * kSlot + kUp + jq * kRoleTiles * 2048 + i * 1024, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)(st + kStDc), 16, lane * 16,
                                                 c * kSlot + kDc, 0, 0);
    };

    // S[t][i] = S[16t + 4q + i][16 j + m16] (wavefront A only)
    f32x4 S[8];
    auto publish_s = [&](int b) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) sbx[b][p][s2][lane] = cat(to_h4(S[2 * s2]), to_h4(S[2 * s2 + 1]));
    };
    if (roleA) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[t][i] = sin ? sin[sbase + (size_t)(16 * t + 4 * q4 + i) * D + 16 * j + m16] : 0.0f;
        publish_s(0);
        if (lane == 0) uflag[p] = 0;
    }
    if (loader) {
        dma(0, 0);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }

    const int ts = a.H * D;
    TOUT* og = static_cast<TOUT*>(a.o);
    const int snap_ic = a.snap ? (int)(a.snap_interval / C) : 1;
    int snap_left = snap_ic - (int)(sa.chunk0 % snap_ic);
    int snap_j = (int)(sa.chunk0 / snap_ic);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // stage c & 1 holds chunk c, sbx[c & 1] its S
        if (loader) {
            if (c + 1 < nch) dma(c + 1, (c + 1) & 1);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the stage is complete before the next barrier
            continue;
        }
        const uint8_t* st = &buf[c & 1][0];
        const h8* nw = reinterpret_cast<const h8*>(st + kNegW);
        const h8* qt = reinterpret_cast<const h8*>(st + kQt);
        const h8* kb = reinterpret_cast<const h8*>(st + kKbT);
        const h8* pm = reinterpret_cast<const h8*>(st + kPm);
        if (roleA) {
            h8 sb[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) sb[s2] = cat(to_h4(S[2 * s2]), to_h4(S[2 * s2 + 1]));
            f32x4 U[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const h4 up = *reinterpret_cast<const h4*>(st + kStUp + ((p * 4 + t) * 64 + lane) * 8);
                U[t] = f32x4{(float)up[0], (float)up[1], (float)up[2], (float)up[3]};
            }
            // U = U' + (-W) S, the operand reads one K step ahead
            h8 an[2][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) an[0][t] = nw[(t * 4 + 0) * 64 + lane];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int cur = s2 & 1, nxt = cur ^ 1;
                if (s2 < 3) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) an[nxt][t] = nw[(t * 4 + s2 + 1) * 64 + lane];
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    U[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(an[cur][t], sb[s2], U[t], 0, 0, 0);
            }
            h8 ak[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ak[i] = kb[i * 64 + lane];  // [t][s] = index t * 2 + s
            h8 ub[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                ub[s2] = cat(to_h4(U[2 * s2]), to_h4(U[2 * s2 + 1]));
                ubx[c & 1][p][s2][lane] = ub[s2];
            }
            // U is in LDS before the counter says so
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            if (lane == 0) __hip_atomic_store(&uflag[p], c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            // S <- Diag(2^b_C) S + Kbar^T U
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 dc = *reinterpret_cast<const f32x4*>(st + kStDc + (16 * t + 4 * q4) * 4);
                f32x4 acc = S[t] * dc;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak[t * 2 + s2], ub[s2], acc, 0, 0, 0);
                S[t] = acc;
            }
            const int64_t cs = seq_s + (sa.chunk0 + c) * C;
            if (a.snap && --snap_left == 0) {
                if (seq_e - cs >= C)
                    store_state_slice(a.snap + (((size_t)n * a.snap_slots + snap_j) * a.H + h) * D * D, S, q4,
                                      16 * j + m16);
                snap_left = snap_ic;
                ++snap_j;
            }
            // S for the next chunk (B read the previous user of this buffer
            // before this chunk's barrier)
            publish_s((c + 1) & 1);
        } else {
            // O^T = S^T Q~^T + U^T P^T: S and U as A operands (the registers of
            // a B operand hold its transpose as an A operand)
            h8 sb[4], aq[2][4], ap[6];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) sb[s2] = sbx[c & 1][p][s2][lane];
#pragma unroll
            for (int t = 0; t < 4; ++t) aq[0][t] = qt[(t * 4 + 0) * 64 + lane];
            f32x4 Ot[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) Ot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int cur = s2 & 1, nxt = cur ^ 1;
                if (s2 < 3) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) aq[nxt][t] = qt[(t * 4 + s2 + 1) * 64 + lane];
                } else {
#pragma unroll
                    for (int i = 0; i < 6; ++i) ap[i] = pm[i * 64 + lane];  // (t, s) with 2s <= t
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    Ot[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sb[s2], aq[cur][t], Ot[t], 0, 0, 0);
            }
            // wait for A's U of this chunk (bounded: a wavefront that never
            // saw it would leave with a wrong output rather than hang)
            for (int spin = 0; spin < (1 << 22); ++spin) {
                if (__hip_atomic_load(&uflag[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > c) break;
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            h8 ub[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) ub[s2] = ubx[c & 1][p][s2][lane];
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int t = i < 2 ? i : 2 + (i - 2) / 2, s2 = i < 2 ? 0 : (i - 2) % 2;
                Ot[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ub[s2], ap[i], Ot[t], 0, 0, 0);
            }
            // lane (token m16 of tile t, q4) holds columns 16j + 4 q4 .. +3;
            // rows past the sequence are dropped by the descriptor range
            const int64_t cs = seq_s + (sa.chunk0 + c) * C;
            const int ntok = (int)min<int64_t>(C, seq_e - cs);
            const rsrc_t ro_ = make_rsrc(og + cs * ts, (int64_t)ntok * ts * (int64_t)sizeof(TOUT));
            const int voff = (m16 * ts + h * D + 16 * j + 4 * q4) * (int)sizeof(TOUT);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 v = a.scale * Ot[t];
                if constexpr (sizeof(TOUT) == 4) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ro_, voff, 16 * t * ts * 4,
                                                           POL);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, to_b4(v)), ro_, voff,
                                                          16 * t * ts * 2, POL);
                }
            }
        }
    }
    if (loader) {
        // no load may still be writing LDS when the workgroup ends
        __builtin_amdgcn_s_waitcnt(0x0f70);
        return;
    }
    if (roleA && sout) {
        int off = 4 * q4 * D + 16 * j + m16;
        asm volatile("" : "+v"(off));
        float* so = sout + sbase + off;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) so[(16 * t + i) * D] = S[t][i];
    }
}

template <typename TOUT, int TPW>
void launch_state(SplitArgs sa, int64_t U, bool stream, hipStream_t s)
{
    constexpr int kColGroups = D / (16 * kStateWaves * TPW);
    sa.map_half = (int)(kColGroups * 8 * ((U + 7) / 8));
    const dim3 gs((unsigned)(sa.map_half * (sa.p.map_M ? 2 : 1))), bs(kStateThreads);
    if (sa.p.map_M) {
        hipLaunchKernelGGL((state_kernel<TOUT, TPW, 0, true>), gs, bs, 0, s, sa);
    } else if constexpr (TPW == 1) {
        // the role-split form: two compute wavefronts per tile. (For the
        // 64-column workgroups a role-split form with four tiles, nine
        // wavefronts and single-buffered hand-overs measured no faster than
        // the two-wavefront form: packed varlen 6.59 against 6.56 ms.)
        static_assert(kStateWaves == kRoleTiles, "the role-split form keeps the 32-column workgroups");
        const dim3 br(kRoleThreads);
        if (stream)
            hipLaunchKernelGGL((state_roles_kernel<TOUT, kStream>), gs, br, 0, s, sa);
        else
            hipLaunchKernelGGL((state_roles_kernel<TOUT, 0>), gs, br, 0, s, sa);
    } else if (stream) {
        hipLaunchKernelGGL((state_kernel<TOUT, TPW, kStream, false>), gs, bs, 0, s, sa);
    } else {
        hipLaunchKernelGGL((state_kernel<TOUT, TPW, 0, false>), gs, bs, 0, s, sa);
    }
}

// A window's workspace up to this size is left to the last-level cache (256
// MiB): the inputs and outputs then go around it (non-temporal hints).
constexpr size_t kStreamWorkspace = (size_t)192 << 20;

}  // namespace

size_t prefill_split_slot_bytes() { return kSlot; }

// ------------------------------------------------------------ static scratch
// The workspace of kda_prefill_noalloc, for callers that cannot allocate
// device memory. Each GPU holds its own copy. In host code `scratch` names a
// host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t prefill_static_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// Intra-pass workgroups per (sequence, head) for a window of nwin chunks with
// `active` (sequence, head) units still running: the grouping that needs the
// fewest rounds of chunks per compute unit (about one workgroup fits a unit),
// the smallest such (every group pays its own first load).
static int intra_groups(int64_t active, int nwin)
{
    int best = 1;
    int64_t best_cost = INT64_MAX;
    for (int g = 1; g <= std::max(nwin, 1); g *= 2) {
        const int64_t cost = (active * g + 255) / 256 * ((nwin + g - 1) / g);
        if (cost < best_cost) {
            best_cost = cost;
            best = g;
        }
    }
    return best;
}

hipError_t launch_prefill_split(const PrefillArgs& a, void* ws, size_t ws_bytes, int64_t max_chunks,
                                const int32_t* cu_host, hipStream_t s)
{
    const int64_t U = (int64_t)a.num_seqs * a.H;
    SplitArgs sa{};
    sa.p = a;
    sa.ws = static_cast<uint8_t*>(ws);
    if (max_chunks <= 0) {
        // every sequence is empty: the state pass only copies the states
        sa.nwin = 1;
    } else if (ws_bytes >= (size_t)(U * max_chunks) * kSlot) {
        sa.nwin = (int)max_chunks;
    } else {
        const size_t carry = (size_t)U * D * D * sizeof(float);
        const int64_t most = std::min<int64_t>(max_chunks, (int64_t)((ws_bytes - carry) / ((size_t)U * kSlot)));
        // as few windows as the workspace allows, about equal in size (a short
        // last window leaves much of the GPU idle), rounded up to a multiple
        // of the intra-pass workgroups per unit (below) so that they all take
        // the same number of chunks
        const int64_t windows = (max_chunks + most - 1) / most;
        const int64_t grp = std::max<int64_t>(1, std::min<int64_t>(most, (256 + U - 1) / U));
        const int64_t even = (max_chunks + windows - 1) / windows;
        sa.nwin = (int)std::min<int64_t>(most, (even + grp - 1) / grp * grp);
        sa.carry = reinterpret_cast<float*>(sa.ws + (size_t)U * most * kSlot);
    }
    const bool stream = (size_t)U * sa.nwin * kSlot <= kStreamWorkspace;
    for (int64_t c0 = 0; c0 < std::max<int64_t>(max_chunks, 1); c0 += sa.nwin) {
        sa.chunk0 = c0;
        // the (sequence, head) units with chunks in this window: packed
        // sequences of different lengths leave fewer in the later windows
        int64_t active = U;
        if (cu_host) {
            int64_t running = 0;
            for (int n = 0; n < a.num_seqs; ++n)
                running += ((int64_t)cu_host[n + 1] - cu_host[n] + 63) / 64 > c0;
            active = running * a.H;
        }
        // intra pass: each workgroup takes every groups-th chunk of its unit's
        // window, its next chunk prefetched; the workgroups of finished units
        // return at once
        sa.groups = intra_groups(active, sa.nwin);
        const dim3 gi((unsigned)(U * sa.groups)), bi(kThreads);
        // state pass: 4 workgroups of 32 columns per state chain while they
        // all fit on the chip at once (one per compute unit; the role-split
        // form, two compute wavefronts per tile), else 2 of 64 columns (each
        // wavefront then carries two tiles through every operand read);
        // segment maps run two chains per unit. Measured: a
        // second round of 32-column workgroups costs more than the wider
        // ones (packed varlen 6.66 against 6.47 ms; one segment's maps, 64
        // heads, 0.070 against 0.064 ms). The two give identical results.
        const int64_t chains = active * (a.map_M ? 2 : 1);
        const bool narrow = chains * 4 <= 256;
        if (max_chunks > 0) {
            if (a.map_M && stream)
                hipLaunchKernelGGL((intra_kernel<bf16_t, kStream, true>), gi, bi, 0, s, sa);
            else if (a.map_M)
                hipLaunchKernelGGL((intra_kernel<bf16_t, 0, true>), gi, bi, 0, s, sa);
            else if (a.gate_f && stream)
                hipLaunchKernelGGL((intra_kernel<bf16_t, kStream, false, true>), gi, bi, 0, s, sa);
            else if (a.gate_f)
                hipLaunchKernelGGL((intra_kernel<bf16_t, 0, false, true>), gi, bi, 0, s, sa);
            else if (stream)
                hipLaunchKernelGGL((intra_kernel<bf16_t, kStream>), gi, bi, 0, s, sa);
            else
                hipLaunchKernelGGL((intra_kernel<bf16_t, 0>), gi, bi, 0, s, sa);
        }
        if (a.out_dtype == F32)
            narrow ? launch_state<float, 1>(sa, U, stream, s) : launch_state<float, 2>(sa, U, stream, s);
        else
            narrow ? launch_state<bf16_t, 1>(sa, U, stream, s) : launch_state<bf16_t, 2>(sa, U, stream, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
