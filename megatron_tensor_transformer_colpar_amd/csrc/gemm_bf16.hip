// bf16 MFMA GEMM for the prefill shapes (M > 32):
//   C[m][n] = sum_k A[m][k] * B[n][k]   (A, B K-contiguous; fp32 accumulate)
// with the epilogue fused: either + bias, GeLU, bf16 store (column-parallel
// up-projection) or an fp32 store (row-parallel partial).
//
// Design for gfx950 (CDNA4), one workgroup per BM x BN output tile, NW waves
// (8 for the large tiles: two per SIMD, so one wave's MFMAs keep issuing
// while the other waits on the issue of its loads; 4 for the small tile):
//  * The waves form a 2 x NW/2 grid, each owning a (BM/2) x (2*BN/NW) block
//    of accumulator tiles on v_mfma_f32_16x16x32_bf16 (it holds a higher
//    clock under the power cap than 32x32x16, although 32x32 tiles need half
//    the LDS fragment reads per flop).  The kernel still takes MF = 32
//    (v_mfma_f32_32x32x16_bf16), which no launch uses.
//  * K advances in BK-wide slices (BK = 64: 128 B per row, or 32) through a
//    ring of S LDS stages filled by direct global->LDS DMA (buffer_load ...
//    lds, 16 B per lane): no staging registers, no ds_write, and S-1 slices
//    in flight.
//  * Within a slice the MFMA fragments of k-step q+1 are read from LDS while
//    the MFMAs of k-step q run.  The barrier that publishes the next slice
//    sits before the last k-step, so the next slice's first fragments are
//    also read under MFMAs, and the slice just finished is refilled at once.
//  * Each 1 KiB DMA block holds 8 rows of 8 16-byte chunks; chunk c of row r
//    lives at slot c ^ op_swz(r), so fragment reads (16 rows, four chunks)
//    spread over all banks.  Rows past M or N read as zero through the
//    buffer resource, so ragged tiles need no branches in the main loop.
//  * The fp32 and bf16 epilogues (partials, activations, gradients) go
//    through LDS, so each store instruction writes whole 128-byte lines.
//  * Waits are explicit (vmcnt for the DMA of the slice about to be used,
//    lgkmcnt(0) so no wave still reads a stage when it is refilled) followed
//    by a bare s_barrier: a __syncthreads() fence would also drain the
//    loads still in flight for later slices.
#include <type_traits>

#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

struct GemmDev {
    const __bf16 *A[kMaxBatch];
    const __bf16 *B[kMaxBatch];
    const __bf16 *bias[kMaxBatch];
    const __bf16 *B2[kMaxBatch];     // gated epilogues: up rows
    const __bf16 *bias2[kMaxBatch];  // gated epilogues: up bias
    __bf16 *aux[kMaxBatch];          // GeLU input: read by the gradient epilogues, written by the GeLU ones
    void *C[kMaxBatch];
    int64_t ldaux;
    int64_t lda, ldb;
    int64_t ldc[kMaxBatch];
    int M, N, K;
    int tiles_m, tiles_n, batch;
    int bands;   // tile order of map_tile_bands (W = tiles_n / 8 columns per XCD)
};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4v;

// Swizzle of the epilogue staging rows (and of 64-byte operand rows, BK =
// 32): chunk c of row r sits at slot c ^ swz(r), spreading 32 consecutive
// rows of one chunk over the banks.
template <int CH>
__device__ __forceinline__ int swz(int row)
{
    if (CH == 8) return (row & 7) ^ ((row >> 3) & 1);         // 128-byte rows
    return ((row >> 1) & 3) ^ ((row >> 3) & 1);                // 64-byte rows
}

// Operand tiles: chunk c of row r sits at slot c ^ op_swz(r).  A 16x16x32
// fragment read (lane l: row l % 16, chunk 4q + l / 16) is conflict-free on
// gfx950 with op_swz(r) = r & 7, and not with swz above, whose flip on row
// bit 3 puts two lanes of the groups the LDS serves together in one bank:
// an LDS read probe of exactly these reads measured 2.45 ns per ds_read_b128
// per CU with r & 7 against 3.88 ns with swz (2.52 ns for 64 lanes reading
// 1 KiB contiguously).
template <int CH>
__device__ __forceinline__ int op_swz(int row)
{
    if (CH == 8) return row & 7;
    return swz<CH>(row);
}

// K-major operand tiles: chunk c of k-row kr sits at slot c ^ kmaj_swz(kr).
// A fragment's transpose reads take four consecutive k-rows per 16-lane
// group, and gfx950 serves the two groups eight k-rows apart together:
// 4(kr & 3) puts one group's four k-rows in four 64-byte spans, 2(kr >> 3 & 1)
// moves the other group's to the other 32 bytes of each, so the 32 lanes
// cover all banks once.  An LDS probe of these reads measured 1.59 ns per
// ds_read_b64_tr_b16 per CU, against 2.19 ns with 4(kr & 3) alone and 1.57
// ns for 64 lanes reading 512 contiguous bytes.  Bits 0, 1 and 3 only: the
// second read of a fragment (four k-rows on) sees the same swizzle.
__device__ __forceinline__ int kmaj_swz(int kr) { return (4 * (kr & 3)) ^ (2 * ((kr >> 3) & 1)); }

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14],
// expcnt[6:4], lgkmcnt[11:8]).
__host__ __device__ constexpr int wait_vm_lgkm0(int vm)
{
    return (vm & 0xF) | (0x7 << 4) | (0x0 << 8) | ((vm >> 4) << 14);
}

template <int BM, int BN, int BK, int S, int NW, int MF = 32>
struct Cfg {
    static constexpr int WN = NW / 2;                  // waves along N (2 along M)
    static constexpr int WTM = BM / 2, WTN = BN / WN;  // wave tile
    static constexpr int TM = WTM / MF, TN = WTN / MF; // MF x MF accumulator tiles per wave
    static constexpr int CH = BK / 8;                  // 16-byte chunks per LDS row
    static constexpr int RB = 64 / CH;                 // rows per 1 KiB DMA block
    static constexpr int KM = MF == 32 ? 16 : 32;      // k per MFMA instruction
    static constexpr int KQ = BK / KM;                 // MFMA k-steps per slice
    static constexpr int CPQ = KM / 8;                 // 16-byte chunks of a row per k-step
    static constexpr int A_LD = BM / RB / NW, B_LD = BN / RB / NW;  // DMA instrs per wave per slice
    static constexpr int LOADS = A_LD + B_LD;          // per thread per slice
    static constexpr int STAGE = (BM + BN) * CH;       // 16-byte slots per stage
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(MF == 16 || MF == 32, "MFMA shape");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles are whole 32x32 blocks");
    static_assert(S >= 2 && S <= 5, "stages");
    static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the DMA layout");
    static_assert((S - 2) * LOADS <= 63, "vmcnt range");
};

// Operand layouts.  K-contiguous (the forward's weights and activations):
// row r of an operand holds its K values, and a tile is BM (or BN) rows of
// BK values.  K-major (LAY 1: B; LAY 2: A and B): element (r, k) sits at
// k * ld + r, as for an activation read along its token axis (the weight
// gradients) or a K-contiguous weight read along its output axis (the input
// gradients).  A K-major tile is BK rows (k) of BM (or BN) values; chunk c
// of k-row kr sits at slot c ^ kmaj_swz(kr), and an MFMA fragment (8 k
// values of one r) is two LDS transpose reads (ds_read_b64_tr_b16: in a
// 16-lane group, lane i gets element i%4 of the 8-byte rows addressed by
// lanes 4j + i/4).  A K-major operand's k-rows are range-checked like rows,
// so K need not be a multiple of BK.
// The order of one 16x16x32 k-step, row by row: TN MFMAs, then the row's
// fragment reads (its A fragment, and B fragment i while i < TN: RA and RB
// LDS reads each, two for a K-major operand's transpose reads), then (RF)
// its share of the refill DMA.
// With single-buffered B fragments (both operands K-major): rows 0 .. TM-2
// are TN MFMAs and the row's A fragment read; the last row reads B fragment
// j of the next k-step right behind MFMA j, then its A fragment.
template <int J, int TN, int RB>
__device__ __forceinline__ void pin_last_row_sb()
{
    if constexpr (J < TN) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
        pin_last_row_sb<J + 1, TN, RB>();
    }
}
template <int I, int TM, int TN, int DPR, int LOADS, bool RF, int RA, int RB>
__device__ __forceinline__ void pin_rows16_sb()
{
    if constexpr (I < TM) {
        if constexpr (I + 1 < TM) {
            __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
        } else {
            pin_last_row_sb<0, TN, RB>();
            __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
        }
        if constexpr (RF && I * DPR < LOADS)
            __builtin_amdgcn_sched_group_barrier(0x020, ((I + 1) * DPR < LOADS ? (I + 1) * DPR : LOADS) - I * DPR, 0);
        pin_rows16_sb<I + 1, TM, TN, DPR, LOADS, RF, RA, RB>();
    }
}
template <int I, int TM, int TN, int DPR, int LOADS, bool RF, int RA = 1, int RB = 1>
__device__ __forceinline__ void pin_rows16()
{
    if constexpr (I < TM) {
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, I < TN ? RA + RB : RA, 0);
        if constexpr (RF && I * DPR < LOADS)
            __builtin_amdgcn_sched_group_barrier(0x020, ((I + 1) * DPR < LOADS ? (I + 1) * DPR : LOADS) - I * DPR, 0);
        pin_rows16<I + 1, TM, TN, DPR, LOADS, RF, RA, RB>();
    }
}

template <int BM, int BN, int BK, int S, int NW, bool IL, int EPI, int LAY, bool NTS, int MF, bool DB>
__global__ void __launch_bounds__(NW * 64) gemm_bf16_kernel(GemmDev g)
{
    using C_ = Cfg<BM, BN, BK, S, NW, MF>;
    constexpr int TM = C_::TM, TN = C_::TN, STAGE = C_::STAGE, CH = C_::CH, RB = C_::RB, KQ = C_::KQ;
    constexpr bool AKM = LAY == 2, BKM = LAY >= 1;   // K-major operands
    static_assert(!(AKM || BKM) || (BK == 64 && BM >= 128 && BN >= 128 && NW % 2 == 0), "K-major tile shape");
    using AccT = typename std::conditional<MF == 32, f32x16, f32x4>::type;
    // Gated: each wave's WTN rows of the B tile are WTN/2 gate rows followed
    // by the matching WTN/2 up rows, so accumulator tiles j and j + TN/2 of a
    // lane hold gate and up of the same output elements; a tile then covers
    // BN/2 output columns.
    constexpr bool GATED = epi_gated(EPI);
    static_assert(!GATED || TN % 2 == 0, "gated tiles pair accumulator tiles within a wave");
    constexpr int BNO = GATED ? BN / 2 : BN;   // output columns per tile
    // LDS.  A stage holds one K slice of both tiles, A rows first.  With DB
    // ("deep B") the two tiles have rings of their own: two A stages and
    // three B stages, five arrays of 32 KiB (all 160 KiB of LDS for the
    // 256 x 256 tile), so a B slice is requested two slices before its use
    // instead of one; every stage is an array of its own, so the compiler
    // never waits for the DMA of one stage before reading another.
    static_assert(!DB || (S == 2 && !epi_gated(EPI)), "deep-B ring shape");
    constexpr int SZ01 = DB ? BM * CH : STAGE, SZB = DB ? BN * CH : STAGE;
    constexpr int SB = DB ? 3 : S;   // B stages (A stages: S)
    __shared__ u32x4 st0[SZ01];
    __shared__ u32x4 st1[SZ01];
    __shared__ u32x4 st2[DB || S > 2 ? SZB : 1];
    __shared__ u32x4 st3[DB || S > 3 ? SZB : 1];
    __shared__ u32x4 st4[DB || S > 4 ? SZB : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    // wave-uniform, kept in an SGPR so the DMA's LDS address (M0) is scalar
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / C_::WN, wn = wave % C_::WN;

    int bt, tile_m, tile_n;
    if (g.bands) {
        map_tile_bands(blockIdx.x, g.tiles_m, g.tiles_n, bt, tile_m, tile_n);
    } else {
        map_tile<8>(blockIdx.x, g.batch, g.tiles_m, g.tiles_n, bt, tile_m, tile_n);
    }
    const int m0 = tile_m * BM, n0 = tile_n * BNO;
    const __bf16 *const Abase = g.A[bt];
    const __bf16 *const Bbase = g.B[bt];
    const __bf16 *const bias_p = g.bias[bt];
    void *const Cbase = g.C[bt];
    const int64_t ldc = g.ldc[bt];
    __bf16 *const aux_p = g.aux[bt];

    const int a_rows = min(BM, g.M - m0), b_rows = min(BNO, g.N - n0);
    // K-contiguous: the tile's rows; K-major: the tile's columns onward, the
    // range ending after the K-th k-row (later k-rows read as zero)
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(AKM ? Abase + m0 : Abase + (int64_t)m0 * g.lda,
                  (uint32_t)(AKM ? ((int64_t)g.K * g.lda - m0) * 2 : (int64_t)a_rows * g.lda * 2));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(BKM ? Bbase + n0 : Bbase + (int64_t)n0 * g.ldb,
                  (uint32_t)(BKM ? ((int64_t)g.K * g.ldb - n0) * 2 : (int64_t)b_rows * g.ldb * 2));
    // (resources are only ever built from pointers: a conditional expression
    // of resource type makes the host compilation drop the kernel's stub)
    const __amdgpu_buffer_rsrc_t rb2 =
        make_rsrc((GATED ? g.B2[bt] : Bbase) + (int64_t)n0 * g.ldb, (uint32_t)((int64_t)b_rows * g.ldb * 2));

    // DMA geometry: instruction j of wave w fills 1 KiB block (NW*j + w),
    // i.e. rows RB(NW*j + w) .. +RB-1; lane L lands in slot L of the block
    // (row L/CH, physical chunk L%CH) and so fetches logical chunk
    // (L%CH) ^ op_swz(row).  The swizzle depends on row bits 0..3 only, so
    // it is the same for every j.
    const int drow = wave * RB + lane / CH;
    const int dchunk = (lane % CH) ^ op_swz<CH>(drow);
    const uint32_t a_voff = (uint32_t)(drow * g.lda * 2 + dchunk * 16);
    const uint32_t b_voff = (uint32_t)(drow * g.ldb * 2 + dchunk * 16);
    const uint32_t a_jstep = (uint32_t)(NW * RB * g.lda * 2), b_jstep = (uint32_t)(NW * RB * g.ldb * 2);
    // K-major tiles: a 1 KiB block is KRA (KRB) k-rows of BM/8 (BN/8)
    // chunks; instruction j of wave w fills block NW*j + w, lane L lands in
    // k-row L/(BM/8) of it, physical chunk L%(BM/8), and fetches the logical
    // chunk the swizzle puts there (j moves the k-row by a multiple of 16,
    // so kmaj_swz does not depend on j).
    constexpr int ACH = BM / 8, BCH = BN / 8, KRA = 64 / ACH, KRB = 64 / BCH;
    static_assert(!AKM || (NW * KRA) % 16 == 0, "K-major A: the DMA step keeps k-row bits 0..3");
    static_assert(!BKM || (NW * KRB) % 16 == 0, "K-major B: the DMA step keeps k-row bits 0..3");
    const int a_krow = wave * KRA + lane / ACH, b_krow = wave * KRB + lane / BCH;
    const uint32_t ak_voff = (uint32_t)((a_krow * g.lda + 8 * ((lane % ACH) ^ kmaj_swz(a_krow))) * 2);
    const uint32_t bk_voff = (uint32_t)((b_krow * g.ldb + 8 * ((lane % BCH) ^ kmaj_swz(b_krow))) * 2);
    const uint32_t ak_jstep = (uint32_t)(NW * KRA * g.lda * 2), bk_jstep = (uint32_t)(NW * KRB * g.ldb * 2);
    const int KT = (AKM || BKM) ? (g.K + BK - 1) / BK : g.K / BK;
    // Gated B rows: instruction j of this wave fills tile rows r0 .. r0+RB-1,
    // r0 = RB(NW*j + wave), all in one half of one wave's WTN rows; they come
    // from output rows ob .. ob+RB-1 of the gate (first half) or up matrix.
    uint32_t gv_off[C_::B_LD];
    bool gv_up[C_::B_LD];
#pragma unroll
    for (int j = 0; j < C_::B_LD; ++j) {
        const int r0 = RB * (NW * j + wave), rr = r0 % C_::WTN;
        gv_up[j] = rr >= C_::WTN / 2;
        const int ob = (r0 / C_::WTN) * (C_::WTN / 2) + rr % (C_::WTN / 2);
        gv_off[j] = (uint32_t)((ob + lane / CH) * g.ldb * 2 + dchunk * 16);
    }

    // The row offset stays in the per-lane voffset, which the buffer range
    // check covers, so rows past M or N read zero; the in-row K offset goes
    // in soffset.  Refills past the last slice re-read the last slice.
    // issue_part(sa, sb, kta, ktb, lo, hi) issues DMA instructions lo .. hi-1
    // of a refill: the A_LD instructions of A slice kta into sa, then the B_LD
    // of B slice ktb into sb (one slice of a shared stage: sb = sa + BM*CH).
    auto issue_part = [&](u32x4 *sa, u32x4 *sb, int kta, int ktb, int lo, int hi) __attribute__((always_inline)) {
        int kt = kta;
        u32x4 *const stage = sa;
        uint32_t koff = (uint32_t)min(kt, KT - 1) * (BK * 2);
#pragma unroll
        for (int j = 0; j < C_::A_LD; ++j) {
            if (j < lo || j >= hi) continue;
            if constexpr (AKM) {
                const uint32_t vo = ak_voff + j * ak_jstep + (uint32_t)min(kt, KT - 1) * (uint32_t)(BK * g.lda * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LDS_PTR(stage + (NW * j + wave) * 64), 16, vo, 0, 0, 0);
            } else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, LDS_PTR(stage + (NW * j + wave) * 64), 16,
                                                        a_voff + j * a_jstep, koff, 0, 0);
        }
        kt = ktb;
        koff = (uint32_t)min(kt, KT - 1) * (BK * 2);
#pragma unroll
        for (int j = 0; j < C_::B_LD; ++j) {
            if (C_::A_LD + j < lo || C_::A_LD + j >= hi) continue;
            if constexpr (BKM) {
                const uint32_t vo = bk_voff + j * bk_jstep + (uint32_t)min(kt, KT - 1) * (uint32_t)(BK * g.ldb * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LDS_PTR(sb + (NW * j + wave) * 64), 16, vo,
                                                        0, 0, 0);
            } else if constexpr (GATED) {
                // the offset goes through a local: an array element passed
                // straight to the builtin also makes the host pass drop the stub
                const uint32_t vo = gv_off[j];
                if (gv_up[j])
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb2, LDS_PTR(sb + (NW * j + wave) * 64), 16,
                                                            vo, koff, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LDS_PTR(sb + (NW * j + wave) * 64), 16,
                                                            vo, koff, 0, 0);
            } else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LDS_PTR(sb + (NW * j + wave) * 64), 16,
                                                        b_voff + j * b_jstep, koff, 0, 0);
        }
    };

    // fragment geometry: lane reads row (lane % MF) of each MF-row tile,
    // K chunk CPQ*q + lane/MF of the slice (32x32x16: 16 k per step, lanes
    // 0-31 and 32-63 take 8 each; 16x16x32: 32 k per step, four groups of 16
    // lanes take 8 each).  The operand swizzle keeps the 16x16x32 reads
    // conflict-free (see op_swz).
    const int frow = lane % MF, fq = lane / MF, fsw = op_swz<CH>(frow);
    const int fhalf = lane >> 5;   // 32x32 tiles: the lane's k half (also its column half in the result)
    const int a_base = (wm * C_::WTM + frow) * CH;
    const int b_base = (BM + wn * C_::WTN + frow) * CH;

    // K-major fragment of MF-row block rb, k-step q, as two transpose reads
    // e4 = 0, 1 (in a 16-lane group, lane i receives element i%4 of the
    // 8-byte pieces addressed by lanes 4j + i/4, j = 0..3: four k-rows of the
    // row i):
    //   32x32x16: lane 32*fhalf + 16*g + i takes row rb + 16g + i, k = 16q +
    //     8*fhalf + 4*e4 + 0..3; lane i addresses k-row +i/4, 8 bytes at
    //     r = rb + 16g + 4*(i%4);
    //   16x16x32: lane 16*kg + i takes row rb + i, k = 32q + 8*kg + 4*e4 +
    //     0..3; lane i addresses k-row +i/4, 8 bytes at r = rb + 4*(i%4).
    // The lane's k-rows have bits 0..1 = trr and bit 3 = its 16-lane group's
    // parity (16x16x32) or its k half (32x32x16); kmaj_swz of those places
    // the 32 lanes of two groups on all banks once.
    const int trr = (lane >> 2) & 3;
    const int tsw = kmaj_swz(trr + 8 * (MF == 32 ? (lane >> 5) & 1 : (lane >> 4) & 1));
    const int tr_chunk = MF == 32 ? 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1) : (lane & 3) >> 1;
    // Byte offsets of the 32-row blocks (their first chunk is a multiple of
    // 4); with 16x16 tiles block i is half i%2 of 32-row block i/2, two
    // chunks on, i.e. the same offset with bit 5 flipped, so the offsets of
    // half the blocks stay in registers.
    constexpr int TRM = MF == 16 ? TM / 2 : TM, TRN = MF == 16 ? TN / 2 : TN;
    int a_tr[TRM], b_tr[TRN];
#pragma unroll
    for (int i = 0; i < TRM; ++i) a_tr[i] = 16 * (((wm * C_::WTM + 32 * i) / 8 + tr_chunk) ^ tsw) + 8 * (lane & 1);
#pragma unroll
    for (int j = 0; j < TRN; ++j) b_tr[j] = 16 * (((wn * C_::WTN + 32 * j) / 8 + tr_chunk) ^ tsw) + 8 * (lane & 1);
    auto a_tro = [&](int i) __attribute__((always_inline)) { return MF == 16 ? a_tr[i >> 1] ^ (32 * (i & 1)) : a_tr[i]; };
    auto b_tro = [&](int j) __attribute__((always_inline)) { return MF == 16 ? b_tr[j >> 1] ^ (32 * (j & 1)) : b_tr[j]; };
    // The reads index the stage in 8-byte elements (every offset here is a
    // multiple of 8): formed as byte offsets, the second read of each pair
    // lost track of which LDS array it reads, and the compiler made it wait
    // for every global->LDS load in flight, the next slices' included.
    auto tr_frag = [&](const u32x4 *region, int rowbytes, int off, int q) __attribute__((always_inline)) {
        const lds_bf16x4v *b8 = reinterpret_cast<const lds_bf16x4v *>(LDS_PTR(region));
        const int k0 = MF == 32 ? 16 * q + 8 * fhalf + trr : 32 * q + 8 * (lane >> 4) + trr;
        const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4v *)(b8 + ((k0 * rowbytes + off) >> 3)));
        const bf16x4v hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4v *)(b8 + (((k0 + 4) * rowbytes + off) >> 3)));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    bf16x8 fa[2][TM], fb[2][TN];
    const int b_off = b_base - BM * CH;   // B fragment offset from the B tile
    // the fragments of k-step q of the A slice at sa and the B slice at sb
    auto read_frags = [&](const u32x4 *sa, const u32x4 *sb, int q, int p) __attribute__((always_inline)) {
        const int slot = (C_::CPQ * q + fq) ^ fsw;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (AKM)
                fa[p][i] = tr_frag(sa, BM * 2, a_tro(i), q);
            else
                fa[p][i] = __builtin_bit_cast(bf16x8, sa[a_base + i * MF * CH + slot]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (BKM)
                fb[p][j] = tr_frag(sb, BN * 2, b_tro(j), q);
            else
                fb[p][j] = __builtin_bit_cast(bf16x8, sb[b_off + j * MF * CH + slot]);
        }
    };

    AccT acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = AccT{};

    // B is the MFMA's first operand, so the result is the tile transposed:
    // lane l ends up with runs of 4 consecutive columns of row l%MF, which
    // the epilogue handles as vectors.  16x16x32 draws less power per flop
    // than 32x32x16: a register-only loop on bf16 data of this kind, two
    // waves per SIMD, sustains 1.97 PFLOP/s at 1972 MHz against 1.77 PFLOP/s
    // at 1767 MHz, both with the matrix cores 95% busy (MI355X, power-capped).
    auto mfmas = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (MF == 32)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[p][j], fa[p][i], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[p][j], fa[p][i], acc[i][j], 0, 0, 0);
            }
    };

    // Each phase issues the next k-step's fragment reads and the current
    // k-step's MFMAs.  sched_group_barriers pin the interleave (the scheduler
    // would otherwise sink each read down to its first use and expose the
    // LDS latency); sched_barrier(0) closes the phase.  In the phase after
    // the barrier the refill DMA of the finished stage is spread between the
    // MFMAs as well, so the matrix pipe never waits for the issue of loads.
    constexpr int NR = TM + TN, NM = TM * TN;
    auto pin_reads = [&]() __attribute__((always_inline)) {
        if (IL) {
            constexpr int per = NM / NR;   // MFMAs per fragment read
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
            }
            if (NM - per * NR > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM - per * NR, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
    };
    auto phase = [&](const u32x4 *sa, const u32x4 *sb, int q, int p_read, int p_mfma) __attribute__((always_inline)) {
        read_frags(sa, sb, q, p_read);
        mfmas(p_mfma);
        pin_reads();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto phase_refill = [&](u32x4 *ra, u32x4 *rb, int kta, int ktb, const u32x4 *sa, const u32x4 *sb, int p_read,
                            int p_mfma) __attribute__((always_inline)) {
        read_frags(sa, sb, 0, p_read);
        issue_part(ra, rb, kta, ktb, 0, C_::LOADS);
        mfmas(p_mfma);
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
        for (int r = 0; r < C_::LOADS; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        if (NM > C_::LOADS) __builtin_amdgcn_sched_group_barrier(0x008, NM - C_::LOADS, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The barrier's wait in every K slice leaves in flight only what was
    // requested after the next slice: with DB the B slice two ahead (each
    // refill requests A before B, so the deeper ring's loads are the
    // youngest), else the S-2 younger slices.
    constexpr int LOOP_WAIT = DB ? C_::B_LD : (S - 2) * C_::LOADS;
    // One K slice, A in ca and B in cb; (na, nb) hold the next slice (its DMA
    // may still be in flight); ca and cb are refilled with A slice kt + S and
    // B slice kt + SB.
    auto slice = [&](u32x4 *ca, u32x4 *cb, const u32x4 *na, const u32x4 *nb, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 1; q < KQ; ++q) phase(ca, cb, q, q & 1, (q - 1) & 1);
        // the next slice landed and every wave is done reading this one
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(LOOP_WAIT));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        phase_refill(ca, cb, kt + S, kt + SB, na, nb, 0, (KQ - 1) & 1);
    };

    // 16x16x32 tiles: a wave's fragments of both buffers would not fit
    // beside its 128 accumulator registers (two waves per SIMD), so the A
    // fragments are single-buffered: A fragment i of the next k-step is read
    // right after the MFMAs of row i (its last use) are issued; the B
    // fragments stay double-buffered, except with both operands K-major
    // (the weight gradients), whose transpose reads need the registers: there
    // B fragment j of the next k-step is read right after the last row's
    // MFMA j (with double-buffered B they spilled 16-20 registers, whose
    // reloads in the main loop waited on the DMA's counter; the backward at
    // the prefill shape took 2096 against 2129 us on 32x32x16 and 2398 us
    // with the spills, bitwise equal).  Each row of MFMAs is followed by its
    // reads and, in the step after the barrier, by its share of the refill
    // DMA; sched_group_barriers pin that order.
    static_assert(MF == 32 || (KQ == 2 && TN <= TM), "16x16x32 main loop shape");
    constexpr int DPR = (C_::LOADS + TM - 1) / TM;   // refill DMA instructions per row
    // step16 reads k-step rq of the A and B slices at ra, rb and (refill)
    // issues A slice kta into fa_st and B slice ktb into fb_st
    auto step16 = [&](auto refill_tag, const u32x4 *ra, const u32x4 *rb, int rq, int pm, int pr, u32x4 *fa_st,
                      u32x4 *fb_st, int kta, int ktb) __attribute__((always_inline)) {
        constexpr bool RF = decltype(refill_tag)::value;
        if constexpr (MF == 16 && AKM && BKM) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i + 1 < TM) {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
                } else {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
                        fb[0][j] = tr_frag(rb, BN * 2, b_tro(j), rq);
                    }
                }
                fa[0][i] = tr_frag(ra, BM * 2, a_tro(i), rq);
                if constexpr (RF)
                    issue_part(fa_st, fb_st, kta, ktb, i * DPR, min((i + 1) * DPR, C_::LOADS));
            }
            pin_rows16_sb<0, TM, TN, DPR, C_::LOADS, RF, 2, 2>();
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (MF == 16) {
            const int slot = (C_::CPQ * rq + fq) ^ fsw;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[pm][j], fa[0][i], acc[i][j], 0, 0, 0);
                if constexpr (AKM)
                    fa[0][i] = tr_frag(ra, BM * 2, a_tro(i), rq);
                else
                    fa[0][i] = __builtin_bit_cast(bf16x8, ra[a_base + i * MF * CH + slot]);
                if (i < TN) {
                    if constexpr (BKM)
                        fb[pr][i] = tr_frag(rb, BN * 2, b_tro(i), rq);
                    else
                        fb[pr][i] = __builtin_bit_cast(bf16x8, rb[b_off + i * MF * CH + slot]);
                }
                if constexpr (RF)
                    issue_part(fa_st, fb_st, kta, ktb, i * DPR, min((i + 1) * DPR, C_::LOADS));
            }
            pin_rows16<0, TM, TN, DPR, C_::LOADS, RF, AKM ? 2 : 1, BKM ? 2 : 1>();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // One K slice, A in ca and B in cb: k-step 0 (reading k-step 1 of the
    // slice), the barrier that publishes the next slice (na, nb), k-step 1
    // (reading k-step 0 of the next slice, refilling ca with A slice kt + S
    // and cb with B slice kt + SB).
    auto slice16 = [&](u32x4 *ca, u32x4 *cb, u32x4 *na, u32x4 *nb, int kt) __attribute__((always_inline)) {
        step16(std::false_type{}, ca, cb, 1, 0, 1, ca, cb, 0, 0);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(LOOP_WAIT));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        step16(std::true_type{}, na, nb, 0, 1, 0, ca, cb, kt + S, kt + SB);
    };

    u32x4 *const ring[5] = {st0, st1, st2, st3, st4};

    // A stage r is ring[r]; B stage r the B part of ring[r], or with DB the
    // array ring[2 + r]
    u32x4 *ring_a[5], *ring_b[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) {
        ring_a[r] = ring[r];
        ring_b[r] = DB ? ring[(2 + r) % 5] : r < S ? ring[r] + BM * CH : ring[r];
    }
    // prologue: A slices 0 .. S-1 and B slices 0 .. SB-1 in flight, slice 0
    // landed and published
    constexpr int PRO = S > SB ? S : SB;
#pragma unroll
    for (int r = 0; r < PRO; ++r)
        issue_part(ring_a[r], ring_b[r], r, r, r < S ? 0 : C_::A_LD, r < SB ? C_::LOADS : C_::A_LD);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(DB ? C_::LOADS + C_::B_LD : (S - 1) * C_::LOADS));
    __builtin_amdgcn_s_barrier();
    if constexpr (MF == 16) {
        // the first k-step's fragments, read in the order step16 reads them,
        // so that the waits the compiler places at the top of the main loop
        // (merged over its entry and its back edge) name the reads they need
        const int slot0 = fq ^ fsw;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (AKM)
                fa[0][i] = tr_frag(ring_a[0], BM * 2, a_tro(i), 0);
            else
                fa[0][i] = __builtin_bit_cast(bf16x8, ring_a[0][a_base + i * MF * CH + slot0]);
            if (i < TN) {
                if constexpr (BKM)
                    fb[0][i] = tr_frag(ring_b[0], BN * 2, b_tro(i), 0);
                else
                    fb[0][i] = __builtin_bit_cast(bf16x8, ring_b[0][b_off + i * MF * CH + slot0]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    } else {
        read_frags(ring_a[0], ring_b[0], 0, 0);
    }
    auto one = [&](int r, int k) __attribute__((always_inline)) {
        if constexpr (MF == 16)
            slice16(ring_a[r % S], ring_b[r % SB], ring_a[(r + 1) % S], ring_b[(r + 1) % SB], k);
        else
            slice(ring_a[r % S], ring_b[r % SB], ring_a[(r + 1) % S], ring_b[(r + 1) % SB], k);
    };
    // unrolled over a whole turn of both rings
    constexpr int U = DB ? 6 : S;
    int kt = 0;
    for (; kt + U <= KT; kt += U) {
#pragma unroll
        for (int r = 0; r < U; ++r) one(r, kt + r);
    }
    // the last KT % U slices, each reached only through the one before it,
    // so the compiler's record of the DMA in flight stays exact (as a row of
    // independent ifs its merged record made every fragment read wait for
    // all loads in flight)
    auto rest = [&](auto self, auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        if constexpr (r + 1 < U) {
            if (kt + r < KT) {
                one(r, kt + r);
                self(self, std::integral_constant<int, r + 1>{});
            }
        }
    };
    rest(rest, std::integral_constant<int, 0>{});
    // drain the clamped refills before the workgroup exits
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

    // Epilogue.  The accumulators are read as runs of 4 consecutive output
    // columns of one row: per 32-row band I of the wave tile (WTM/32 bands)
    // a lane holds RUNS = WTN/8 runs, run u covering band row run_row(u) and
    // columns 8*run_chunk(u) + 4*run_half(u) .. +3 of the wave tile, i.e.
    // half run_half(u) of 16-byte bf16 chunk run_chunk(u) of that row.
    //   32x32 tiles: run u = 4j + q is acc[I][j][4q .. 4q+3], row lane%32,
    //                columns 32j + 8q + 4(lane/32);
    //   16x16 tiles: run u = a*TN + j is acc[2I + a][j], row 16a + lane%16,
    //                columns 16j + 4(lane/16).
    // Every epilogue regroups the runs through LDS into whole-line stores.
    constexpr int RUNS = C_::WTN / 8, BANDS = C_::WTM / 32;
    auto run = [&](int I, int u) __attribute__((always_inline)) {
        if constexpr (MF == 32) {
            const int j = u / 4, q = u % 4;
            return f32x4{acc[I][j][4 * q], acc[I][j][4 * q + 1], acc[I][j][4 * q + 2], acc[I][j][4 * q + 3]};
        } else {
            return acc[2 * I + u / TN][u % TN];
        }
    };
    auto run_row = [&](int u) __attribute__((always_inline)) {
        return MF == 32 ? (lane & 31) : 16 * (u / TN) + (lane & 15);
    };
    auto run_chunk = [&](int u) __attribute__((always_inline)) {
        return MF == 32 ? u : 2 * (u % TN) + (lane >> 5);
    };
    auto run_half = [&](int u) __attribute__((always_inline)) {
        return MF == 32 ? (lane >> 5) : ((lane >> 4) & 1);
    };
    const bool full = (m0 + BM <= g.M) && (n0 + BNO <= g.N);
    // 4 bias values at column n: zeros past N or without a bias (a resource
    // of 0 bytes), through the buffer range check, so the loads of every run
    // are issued together with no branch between them
    auto bias_rsrc = [&](const __bf16 *bp) __attribute__((always_inline)) {
        return make_rsrc(bp, bp ? (uint32_t)g.N * 2 : 0u);
    };
    auto load_bias4 = [&](__amdgpu_buffer_rsrc_t rbias, int n) __attribute__((always_inline)) {
        const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rbias, n * 2, 0, 0));
        return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xFFFF0000u),
                     __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xFFFF0000u)};
    };
    if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_ACC_F32) {
        // fp32 output leaves through LDS, one 32x32 block (a band's columns
        // 32J .. 32J+31) at a time per wave (4 KiB each, inside stage 0), so
        // that every store instruction writes 8 rows x 128 contiguous bytes,
        // i.e. whole lines.  Stored straight from the accumulators, an
        // instruction wrote 32 bytes in each of 32 rows; on the 4-shard
        // row-parallel launch at 2048 tokens that took 261 us against 247 us
        // like this.  Rows of the staging block are 8 chunks of 4 floats;
        // chunk c of row r sits at slot c ^ swz(r), which keeps both the
        // column-wise write and the row-wise read conflict-free.  A wave's
        // LDS operations complete in issue order, so no wait separates its
        // writes from its reads or one block's reads from the next block's
        // writes.
        static_assert(NW * 32 * 32 * 4 <= SZ01 * 16, "epilogue staging area");
        __syncthreads();   // every wave is done reading the last slice
        float *const stg = reinterpret_cast<float *>(st0) + wave * 32 * 32;
        const int mw = m0 + wm * C_::WTM, nw = n0 + wn * C_::WTN;
        const int rrow = lane >> 3, rch = lane & 7;
#pragma unroll
        for (int I = 0; I < BANDS; ++I) {
#pragma unroll
            for (int J = 0; J < C_::WTN / 32; ++J) {
                // the 4 runs of this lane in block J: 32x32 tiles u = 4J .. 4J+3;
                // 16x16 tiles tile columns 2J, 2J+1 of both 16-row halves
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int u = MF == 32 ? 4 * J + w : (w / 2) * TN + 2 * J + (w % 2);
                    const int r = run_row(u), c = 2 * run_chunk(u) + run_half(u) - 8 * J;
                    *reinterpret_cast<f32x4 *>(stg + r * 32 + 4 * (c ^ swz<8>(r))) = run(I, u);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int r = 8 * rr + rrow;
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(stg + r * 32 + 4 * (rch ^ swz<8>(r)));
                    const int m = mw + 32 * I + r, n = nw + 32 * J + 4 * rch;
                    if (full || (m < g.M && n < g.N)) {
                        f32x4 *const c = reinterpret_cast<f32x4 *>(static_cast<float *>(Cbase) + (int64_t)m * ldc + n);
                        if constexpr (EPI == EPI_ACC_F32)
                            *c = *c + x;   // accumulate (weight gradients over micro-batches)
                        else if constexpr (NTS)
                            __builtin_nontemporal_store(x, c);   // streamed past the caches (see launch_cfg)
                        else
                            *c = x;
                    }
                }
            }
        }
    } else if constexpr (GATED) {
        // The gated tile (BM x BNO bf16) is staged whole in stage 0, then
        // stored as whole rows.  A wave's WTN accumulator columns are WTN/2
        // gate columns followed by the matching WTN/2 up columns, so gate run
        // u (in the first half) pairs with up run u + RUNS/2 (32x32 tiles) or
        // u + TN/2 (16x16 tiles); the pair gives output row wm*WTM + 32I +
        // run_row(u), chunk wn*WTN/16 + run_chunk(u), half run_half(u).
        // Chunk c of row r sits at slot c ^ (r % CPL), so the 8-byte writes
        // of one instruction and the row-wise 16-byte reads spread over the
        // banks.
        constexpr int CPL = BNO / 8;   // 16-byte chunks per output row
        static_assert(BM * BNO * 2 <= SZ01 * 16, "gated staging area");
        static_assert((BM * CPL) % (64 * NW) == 0 && 64 % CPL == 0, "gated drain geometry");
        const __bf16 *const bias2_p = g.bias2[bt];
        __syncthreads();   // every wave is done reading the last slice
#pragma unroll
        for (int u = 0; u < RUNS; ++u) {
            const bool gate = MF == 32 ? u < RUNS / 2 : (u % TN) < TN / 2;
            if (!gate) continue;
            const int uu = MF == 32 ? u + RUNS / 2 : u + TN / 2;
            const int c = wn * (C_::WTN / 16) + run_chunk(u);
            const int n = n0 + 8 * c + 4 * run_half(u);
            const f32x4 bgv = load_bias4(bias_rsrc(bias_p), n), buv = load_bias4(bias_rsrc(bias2_p), n);
#pragma unroll
            for (int I = 0; I < BANDS; ++I) {
                const int r = wm * C_::WTM + 32 * I + run_row(u);
                const f32x4 ga = run(I, u) + bgv, up = run(I, uu) + buv;
                const bf16x4 y = {(__bf16)(act<EPI>(ga[0]) * up[0]), (__bf16)(act<EPI>(ga[1]) * up[1]),
                                  (__bf16)(act<EPI>(ga[2]) * up[2]), (__bf16)(act<EPI>(ga[3]) * up[3])};
                reinterpret_cast<u32x2 *>(st0 + r * CPL + (c ^ (r % CPL)))[run_half(u)] = __builtin_bit_cast(u32x2, y);
            }
        }
        __syncthreads();
        constexpr int RPI = 64 / CPL;   // output rows per store instruction
#pragma unroll
        for (int k = 0; k < BM * CPL / (64 * NW); ++k) {
            const int r = (k * NW + wave) * RPI + lane / CPL, c = lane % CPL;
            const u32x4 v = st0[r * CPL + (c ^ (r % CPL))];
            const int m = m0 + r, n = n0 + 8 * c;
            if (full || (m < g.M && n < g.N))
                *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(Cbase) + (int64_t)m * ldc + n) = v;
        }
    } else {
        // bf16 output (and the kept GeLU input) leaves through LDS like the
        // fp32 output: a wave stages its 32 x WTN block of one band (a lane
        // puts run u into half run_half(u) of chunk run_chunk(u) of row
        // run_row(u)), then reads it back row-wise, so a store instruction
        // writes 64/CHR rows x CHR*16 contiguous bytes: whole 128-byte lines
        // when WTN = 64.
        constexpr int CHR = RUNS, RPI = 64 / CHR;
        static_assert(NW * 32 * CHR <= SZ01, "epilogue staging area");
        __syncthreads();   // every wave is done reading the last slice
        u32x4 *const stg = st0 + wave * 32 * CHR;
        const int mw = m0 + wm * C_::WTM, nw = n0 + wn * C_::WTN;
        f32x4 bias[RUNS];
#pragma unroll
        for (int u = 0; u < RUNS; ++u)
            bias[u] = epi_has_bias(EPI) ? load_bias4(bias_rsrc(bias_p), nw + 8 * run_chunk(u) + 4 * run_half(u)) : f32x4{};
        auto put = [&](int u, f32x4 v) __attribute__((always_inline)) {
            const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            const int r = run_row(u);
            reinterpret_cast<u32x2 *>(stg + r * CHR + (run_chunk(u) ^ swz<CHR>(r)))[run_half(u)] =
                __builtin_bit_cast(u32x2, b);
        };
        auto drain = [&](__bf16 *dst, int64_t ld, int I) __attribute__((always_inline)) {
#pragma unroll
            for (int rr = 0; rr < CHR / 2; ++rr) {
                const int r = RPI * rr + lane / CHR, c = lane % CHR;
                const u32x4 v = stg[r * CHR + (c ^ swz<CHR>(r))];
                const int m = mw + 32 * I + r, n = nw + 8 * c;
                if (full || (m < g.M && n < g.N)) *reinterpret_cast<u32x4 *>(dst + (int64_t)m * ld + n) = v;
            }
        };
#pragma unroll
        for (int I = 0; I < BANDS; ++I) {
            if constexpr (epi_act_grad(EPI)) {
                // gradient at the GeLU input: x * g'(u), u the saved GeLU input.
                // u's rows arrive the way the output leaves: whole lines,
                // row-wise into the slot, then each lane takes its runs (read
                // straight into the accumulator layout, a load touched 16 bytes
                // in each of 32 rows; dU at 2048 tokens 69.6 -> 68.7 us)
                bf16x4 uv[RUNS];
#pragma unroll
                for (int rr = 0; rr < CHR / 2; ++rr) {
                    const int r = RPI * rr + lane / CHR, c = lane % CHR;
                    const int mr = mw + 32 * I + r, n = nw + 8 * c;
                    u32x4 v = {};
                    if (full || (mr < g.M && n < g.N))
                        v = *reinterpret_cast<const u32x4 *>(aux_p + (int64_t)mr * g.ldaux + n);
                    stg[r * CHR + (c ^ swz<CHR>(r))] = v;
                }
#pragma unroll
                for (int u = 0; u < RUNS; ++u) {
                    const int r = run_row(u);
                    uv[u] = __builtin_bit_cast(
                        bf16x4, reinterpret_cast<const u32x2 *>(stg + r * CHR + (run_chunk(u) ^ swz<CHR>(r)))[run_half(u)]);
                }
#pragma unroll
                for (int u = 0; u < RUNS; ++u) {
                    const f32x4 x = run(I, u);
                    put(u, f32x4{x[0] * act_grad<EPI>((float)uv[u][0]), x[1] * act_grad<EPI>((float)uv[u][1]),
                                 x[2] * act_grad<EPI>((float)uv[u][2]), x[3] * act_grad<EPI>((float)uv[u][3])});
                }
                drain(static_cast<__bf16 *>(Cbase), ldc, I);
            } else {
                if (aux_p) {   // keep the GeLU input for the backward pass
#pragma unroll
                    for (int u = 0; u < RUNS; ++u) put(u, run(I, u) + bias[u]);
                    drain(aux_p, g.ldaux, I);
                }
#pragma unroll
                for (int u = 0; u < RUNS; ++u) {
                    const f32x4 x = run(I, u) + bias[u];
                    put(u, f32x4{act<EPI>(x[0]), act<EPI>(x[1]), act<EPI>(x[2]), act<EPI>(x[3])});
                }
                drain(static_cast<__bf16 *>(Cbase), ldc, I);
            }
        }
    }
}

template <int BM, int BN, int BK, int S, int NW, bool IL, int EPI, int LAY, bool NTS = false, bool DB = false>
hipError_t launch_one(const GemmArgs &a, hipStream_t s)
{
    GemmDev g;
    for (int b = 0; b < kMaxBatch; ++b) {
        const int src = b < a.batch ? b : 0;
        g.A[b] = static_cast<const __bf16 *>(a.A[src]);
        g.B[b] = static_cast<const __bf16 *>(a.B[src]);
        g.bias[b] = static_cast<const __bf16 *>(a.bias[src]);
        g.B2[b] = static_cast<const __bf16 *>(a.B2[src]);
        g.bias2[b] = static_cast<const __bf16 *>(a.bias2[src]);
        g.aux[b] = static_cast<__bf16 *>(a.aux[src]);
        g.C[b] = a.C[src];
    }
    g.lda = a.lda;
    g.ldb = a.ldb;
    g.ldaux = a.ldaux;
    for (int b = 0; b < kMaxBatch; ++b) g.ldc[b] = ldc_of(a, b < a.batch ? b : 0);
    g.M = (int)a.M;
    g.N = (int)a.N;
    g.K = (int)a.K;
    g.batch = a.batch;
    constexpr int BNO = epi_gated(EPI) ? BN / 2 : BN;
    g.tiles_m = (int)((a.M + BM - 1) / BM);
    g.tiles_n = (int)((a.N + BNO - 1) / BNO);
    // Row-parallel partials on the 256 x 256 tile with at least 4 tile
    // columns per XCD take the band order: alternating with the column-
    // parallel launch at the prefill shape (whose operands push W2 out of
    // the last-level cache), the pair took 770.3 instead of 785.3 us,
    // bit-identical.
    g.bands = EPI == EPI_STORE_F32 && LAY == 0 && BM == 256 && BN == 256 && g.tiles_n % 8 == 0 && g.tiles_n >= 32;
    const dim3 grid((unsigned)(g.batch * g.tiles_m * g.tiles_n)), block(NW * 64);
    // 16x16x32 MFMAs draw less power per flop than 32x32x16 and hold a
    // higher clock under the power cap: the input gradients (one K-major
    // operand) took the backward at the prefill shape from 2158 to 2111 us
    // with them, bitwise equal, and the weight gradients (single-buffered B
    // fragments, see the main loop) from 2129 to 2096 us.  Accumulating
    // weight gradients followed once the conflict-free K-major layout freed
    // the registers their epilogue needs: 2180.2 -> 2149.4 us for the
    // forward and the accumulating backward at the prefill shape, bitwise
    // equal.
    constexpr int MF = 16;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, S, NW, IL, EPI, LAY, NTS, MF, DB>), grid, block, 0, s, g);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int S, int NW, bool IL>
hipError_t launch_cfg(const GemmArgs &a, Epilogue epi, hipStream_t s)
{
    constexpr bool gated_ok = Cfg<BM, BN, BK, S, NW, 16>::TN % 2 == 0 && Cfg<BM, BN, BK, S, NW, 16>::WTN >= 64;
    // A launch whose fp32 output exceeds half the 256 MB last-level cache
    // (a row-parallel partial at 8192 tokens is 256 MiB) streams it out with
    // non-temporal stores: it cannot stay cached for its consumer anyway,
    // and cached stores leave the tiles' epilogues waiting on write-backs
    // (on the prefill shape the row-parallel launch took 418-439 us against
    // 450-474 us with cached stores, alternating builds on two boxes).
    // Smaller outputs, such as the 2048-token block's four partials (128 MiB)
    // that its reduce reads right after, stay cached.
    const bool stream = (int64_t)a.batch * a.M * a.N * 4 > (int64_t(128) << 20);
    // The 256 x 256 forward tile takes a third B stage in the LDS it leaves
    // free (the gated epilogue needs a 64 KiB staging area and keeps two
    // shared stages).  A weight panel that is not in the last-level cache
    // (the launch before streamed other operands through it) then has two
    // slices to arrive instead of one.
    constexpr bool DBC = BM == 256 && BN == 256 && BK == 64 && S == 2;
    if (a.layout == LAYOUT_B_KMAJOR) {   // input gradients
        switch (epi) {
        case EPI_STORE_F32:
            return stream ? launch_one<BM, BN, BK, S, NW, IL, EPI_STORE_F32, 1, true>(a, s)
                          : launch_one<BM, BN, BK, S, NW, IL, EPI_STORE_F32, 1>(a, s);
        case EPI_BIAS: return launch_one<BM, BN, BK, S, NW, IL, EPI_BIAS, 1>(a, s);
        case EPI_GELU_GRAD_TANH: return launch_one<BM, BN, BK, S, NW, IL, EPI_GELU_GRAD_TANH, 1>(a, s);
        case EPI_GELU_GRAD_ERF: return launch_one<BM, BN, BK, S, NW, IL, EPI_GELU_GRAD_ERF, 1>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    if (a.layout == LAYOUT_AB_KMAJOR) {  // weight gradients
        switch (epi) {
        case EPI_STORE_F32: return launch_one<BM, BN, BK, S, NW, IL, EPI_STORE_F32, 2>(a, s);
        case EPI_ACC_F32: return launch_one<BM, BN, BK, S, NW, IL, EPI_ACC_F32, 2>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (epi) {
    case EPI_BIAS_GELU: return launch_one<BM, BN, BK, S, NW, IL, EPI_BIAS_GELU, 0, false, DBC>(a, s);
    case EPI_STORE_F32:
        return stream ? launch_one<BM, BN, BK, S, NW, IL, EPI_STORE_F32, 0, true, DBC>(a, s)
                      : launch_one<BM, BN, BK, S, NW, IL, EPI_STORE_F32, 0, false, DBC>(a, s);
    case EPI_BIAS_GELU_ERF: return launch_one<BM, BN, BK, S, NW, IL, EPI_BIAS_GELU_ERF, 0, false, DBC>(a, s);
    case EPI_BIAS: return launch_one<BM, BN, BK, S, NW, IL, EPI_BIAS, 0, false, DBC>(a, s);
    case EPI_GATED_TANH:
        if constexpr (gated_ok) return launch_one<BM, BN, BK, S, NW, IL, EPI_GATED_TANH, 0>(a, s);
        break;
    case EPI_GATED_ERF:
        if constexpr (gated_ok) return launch_one<BM, BN, BK, S, NW, IL, EPI_GATED_ERF, 0>(a, s);
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs &a, Epilogue epi, int num_cu, hipStream_t s)
{
    // Largest tile that still gives every CU at least one workgroup.
    auto tiles = [&](int bm, int bn) __attribute__((always_inline)) {
        return a.batch * ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    };
    if (epi_gated(epi)) {
        // a gated tile writes half its width; the 256x128 shape has a single
        // 32-column accumulator tile per wave and cannot pair gate with up
        if (tiles(256, 128) >= num_cu) return launch_cfg<256, 256, 64, 2, 8, true>(a, epi, s);
        return launch_cfg<128, 128, 64, 3, 4, true>(a, epi, s);
    }
    if (tiles(256, 256) >= num_cu) return launch_cfg<256, 256, 64, 2, 8, true>(a, epi, s);
    if (tiles(256, 128) >= num_cu) return launch_cfg<256, 128, 64, 3, 8, true>(a, epi, s);
    return launch_cfg<128, 128, 64, 3, 4, true>(a, epi, s);
}

}  // namespace tpk
