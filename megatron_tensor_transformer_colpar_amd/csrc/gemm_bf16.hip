// bf16 MFMA GEMM for the prefill shapes (M > 32):
//   C[m][n] = sum_k A[m][k] * B[n][k]   (A, B K-contiguous; fp32 accumulate)
// with the epilogue fused: either + bias, GeLU, bf16 store (column-parallel
// up-projection) or an fp32 store (row-parallel partial).
//
// Design for gfx950 (CDNA4):
//  * v_mfma_f32_32x32x16_bf16: each wave owns a (BM/WM) x (BN/WN) block of
//    32x32 accumulator tiles; 32x32 tiles need half the LDS fragment traffic
//    of 16x16 tiles per flop.
//  * K is staged through LDS in 64-wide slices (128 B per row), double
//    buffered; global -> register loads of slice k+1 are issued before the
//    MFMAs of slice k and written to the other LDS buffer after them, so one
//    barrier per slice suffices.
//  * Global loads are 16 B per lane through buffer resources rooted at the
//    tile: rows past M or N read as zero, no clamping or branches.
//  * LDS rows are 8 chunks of 16 B; chunk c of row r lives at slot
//    c ^ swz(r), so the 32 rows a fragment read touches hit distinct banks.
#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

constexpr int BK = 64;

struct GemmDev {
    const __bf16 *A;
    const __bf16 *B;
    const __bf16 *bias;
    void *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_kernel(GemmDev g)
{
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA tiles per wave
    constexpr int RPI = NT / 8;                  // tile rows per load instruction
    constexpr int A_LD = BM / RPI, B_LD = BN / RPI;
    constexpr int STAGE = (BM + BN) * 8;         // 16-byte slots per LDS stage
    static_assert(TM >= 1 && TN >= 1 && A_LD >= 1 && B_LD >= 1, "tile shape");
    static_assert(RPI % 16 == 0, "load rows must keep the swizzle phase");

    __shared__ u32x4 smem[2 * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tile_m, tile_n;
    map_tile<8>(blockIdx.x, g.tiles_m, g.tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int a_rows = min(BM, g.M - m0), b_rows = min(BN, g.N - n0);
    const __amdgpu_buffer_rsrc_t ra_src =
        make_rsrc(g.A + (int64_t)m0 * g.lda, (uint32_t)((int64_t)a_rows * g.lda * 2));
    const __amdgpu_buffer_rsrc_t rb_src =
        make_rsrc(g.B + (int64_t)n0 * g.ldb, (uint32_t)((int64_t)b_rows * g.ldb * 2));

    // loader geometry: thread t moves chunk (t & 7) of rows (t >> 3) + j*RPI
    const int lrow = t >> 3, lkc = t & 7;
    const int lslot = lrow * 8 + (lkc ^ swz(lrow));
    const uint32_t a_voff = (uint32_t)(lrow * g.lda * 2 + lkc * 16);
    const uint32_t b_voff = (uint32_t)(lrow * g.ldb * 2 + lkc * 16);
    const uint32_t a_step = (uint32_t)(RPI * g.lda * 2), b_step = (uint32_t)(RPI * g.ldb * 2);

    u32x4 ra[A_LD], rb[B_LD];
    auto gload = [&](int kt) {
        const uint32_t soff = (uint32_t)kt * (BK * 2);
#pragma unroll
        for (int j = 0; j < A_LD; ++j) ra[j] = buf_load16(ra_src, a_voff + j * a_step, soff);
#pragma unroll
        for (int j = 0; j < B_LD; ++j) rb[j] = buf_load16(rb_src, b_voff + j * b_step, soff);
    };
    auto sstore = [&](int buf) {
        u32x4 *s = smem + buf * STAGE;
#pragma unroll
        for (int j = 0; j < A_LD; ++j) s[lslot + j * RPI * 8] = ra[j];
#pragma unroll
        for (int j = 0; j < B_LD; ++j) s[BM * 8 + lslot + j * RPI * 8] = rb[j];
    };

    // fragment geometry: lane reads row (lane & 31) of each 32-row tile,
    // K chunk 2*s + (lane >> 5) of the 64-wide slice
    const int frow = lane & 31, fhalf = lane >> 5, fsw = swz(frow);
    const int a_base = (wm * WTM + frow) * 8;
    const int b_base = (BM + wn * WTN + frow) * 8;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    const int KT = g.K / BK;
    gload(0);
    sstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const u32x4 *s = smem + cur * STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int slot = (ks * 2 + fhalf) ^ fsw;
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = __builtin_bit_cast(bf16x8, s[a_base + i * 32 * 8 + slot]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8, s[b_base + j * 32 * 8 + slot]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: accumulator element v of tile (i, j) is
    //   row 8*(v/4) + 4*(lane/32) + v%4, column lane%32
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + frow;
        if (n >= g.N) continue;
        float b = 0.0f;
        if (EPI == EPI_BIAS_GELU && g.bias) b = (float)g.bias[n];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fhalf + (v & 3);
                if (m >= g.M) continue;
                const float x = acc[i][j][v];
                if (EPI == EPI_BIAS_GELU) {
                    static_cast<__bf16 *>(g.C)[(int64_t)m * g.ldc + n] = (__bf16)gelu_tanh(x + b);
                } else {
                    static_cast<float *>(g.C)[(int64_t)m * g.ldc + n] = x;
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs &a, Epilogue epi, hipStream_t s)
{
    GemmDev g;
    g.A = static_cast<const __bf16 *>(a.A);
    g.B = static_cast<const __bf16 *>(a.B);
    g.bias = static_cast<const __bf16 *>(a.bias);
    g.C = a.C;
    g.lda = a.lda;
    g.ldb = a.ldb;
    g.ldc = a.ldc;
    g.M = (int)a.M;
    g.N = (int)a.N;
    g.K = (int)a.K;
    g.tiles_m = (int)((a.M + BM - 1) / BM);
    g.tiles_n = (int)((a.N + BN - 1) / BN);
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(WM * WN * 64);
    if (epi == EPI_BIAS_GELU)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_BIAS_GELU>), grid, block, 0, s, g);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE_F32>), grid, block, 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs &a, Epilogue epi, int num_cu, hipStream_t s)
{
    // Largest tile that still gives every CU at least one workgroup.
    auto tiles = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    if (tiles(256, 256) >= num_cu) return launch_cfg<256, 256, 2, 2>(a, epi, s);
    if (tiles(256, 128) >= num_cu) return launch_cfg<256, 128, 2, 2>(a, epi, s);
    return launch_cfg<128, 128, 2, 2>(a, epi, s);
}

}  // namespace tpk
