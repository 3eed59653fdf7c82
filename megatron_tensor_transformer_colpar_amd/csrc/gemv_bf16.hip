// bf16 skinny-M path (decode, M <= 32):
//   C[m][n] = sum_k X[m][k] * W[n][k]
// At decode the weights are read once and the tokens are few, so the kernel
// is a weight stream: it is bound by HBM bandwidth, and the few tokens ride
// along in MFMA tiles padded to 16 tokens (the MFMA units have orders of
// magnitude of headroom at this intensity, VALU would not at M = 32).
//
// Layout: a workgroup owns 16 weight rows [n0, n0+16) and KS (1, 4 or 8)
// waves; wave w streams the K range [w*K/KS, (w+1)*K/KS) of those rows and
// multiplies it with v_mfma_f32_16x16x32_bf16 against 16-token tiles of X
// (tokens past M read as zero through the buffer resource).  The KS partial
// tiles are then summed in LDS in fixed order (deterministic, no atomics)
// and the epilogue (bias + GeLU -> bf16, or fp32) is applied.  Two stream
// kernels: gemv_seg_kernel (contiguous 256-byte row segments per load,
// regrouped through LDS) whenever each wave's range is a multiple of 128
// elements, else gemv_bf16_kernel (16 rows x 64 bytes per load straight into
// the fragments).
#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

struct GemvDev {
    const __bf16 *X[kMaxBatch];
    const __bf16 *W[kMaxBatch];
    const __bf16 *bias[kMaxBatch];
    const __bf16 *W2[kMaxBatch];     // gated epilogues: up rows
    const __bf16 *bias2[kMaxBatch];  // gated epilogues: up bias
    void *C[kMaxBatch];
    int64_t ldx, ldw;
    int64_t ldc[kMaxBatch];
    int M, N, K;
    int batch;
};

// NT loads (cache policy "nt") for the weight stream, which is read once,
// so the reused token rows stay resident in L2.
constexpr int kStreamPolicy = 2;

// Output element idx (< MT*256) of a block, from the KS partial tiles in
// LDS summed in fixed order.  Accumulator element v of lane l, token tile mt
// is weight row 4*(l/16) + v, token mt*16 + l%16.  Plain blocks are 16
// output columns from n0; gated blocks are 8 gate rows then the 8 matching
// up rows, i.e. 8 output columns from n0, and only lanes l < 32 (rows 0..7)
// write, pairing with the up sum at idx + 32 (row + 8).
template <int EPI, int MT, int KS>
__device__ __forceinline__ void gemv_store(const GemvDev &g, int bt, int n0, int idx, const float (*red)[MT * 4 * 64])
{
    const int l = idx & 63, v = (idx >> 6) & 3, mt = idx >> 8;
    const int m = mt * 16 + (l & 15);
    if (m >= g.M) return;
    auto sum = [&](int k) __attribute__((always_inline)) {
        float s = red[0][k];
#pragma unroll
        for (int j = 1; j < KS; ++j) s += red[j][k];
        return s;
    };
    if constexpr (epi_gated(EPI)) {
        if (l >= 32) return;
        const int n = n0 + 4 * (l >> 4) + v;
        const float bg = g.bias[bt] ? (float)g.bias[bt][n] : 0.0f;
        const float bu = g.bias2[bt] ? (float)g.bias2[bt][n] : 0.0f;
        const float y = act<EPI>(sum(idx) + bg) * (sum(idx + 32) + bu);
        static_cast<__bf16 *>(g.C[bt])[(int64_t)m * g.ldc[bt] + n] = (__bf16)y;
    } else {
        const int n = n0 + 4 * (l >> 4) + v;
        const float s = sum(idx);
        if (EPI == EPI_STORE_F32) {
            static_cast<float *>(g.C[bt])[(int64_t)m * g.ldc[bt] + n] = s;
        } else {
            const float b = g.bias[bt] ? (float)g.bias[bt][n] : 0.0f;
            static_cast<__bf16 *>(g.C[bt])[(int64_t)m * g.ldc[bt] + n] = (__bf16)act<EPI>(s + b);
        }
    }
}

template <int EPI, int MT, int KS, int CHUNK>
__global__ void __launch_bounds__(KS * 64) gemv_bf16_kernel(GemvDev g)
{
    __shared__ float red[KS][MT * 4 * 64];

    constexpr bool GATED = epi_gated(EPI);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int n0 = blockIdx.x * (GATED ? 8 : 16);   // first output column
    const int bt = blockIdx.y;   // batch entry (TP shard)
    const __bf16 *const Xb = g.X[bt];
    const __bf16 *const Wb = g.W[bt];
    const int Kw = g.K / KS;
    const int kbeg = w * Kw;

    // gated: rows 0..7 of the block are gate rows, 8..15 the up rows
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(Wb + (int64_t)n0 * g.ldw, (uint32_t)((GATED ? 8 : 16) * g.ldw * 2));
    const __amdgpu_buffer_rsrc_t wsrc2 = make_rsrc((GATED ? g.W2[bt] : Wb) + (int64_t)n0 * g.ldw,
                                                   (uint32_t)((GATED ? 8 : 16) * g.ldw * 2));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(Xb, (uint32_t)((int64_t)g.M * g.ldx * 2));

    // lane geometry of the 16x16x32 MFMA operands: row (lane & 15), K chunk
    // (lane >> 4) of 8 elements
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    const uint32_t w_voff = (uint32_t)((r16 * g.ldw + kbeg + kq) * 2);
    // gated: a gate lane's offset in the up matrix, and an up lane's in the
    // gate matrix, lie past the 8-row range and read zero (and no memory),
    // so the OR of the two loads is the lane's own row
    const uint32_t w_voff2 = (uint32_t)(((r16 - 8) * g.ldw + kbeg + kq) * 2);
    uint32_t x_voff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) x_voff[mt] = (uint32_t)(((mt * 16 + r16) * g.ldx + kbeg + kq) * 2);

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{};

    // Every load of a chunk is issued before its first MFMA, so a wave keeps
    // CHUNK KiB of weights in flight and the KS waves of the CU together
    // cover the HBM latency.
    for (int k = 0; k < Kw; k += 32 * CHUNK) {
        u32x4 wv[CHUNK], xv[CHUNK][MT];
        const uint32_t soff = (uint32_t)k * 2;
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
            wv[c] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, (int)(w_voff + c * 64), (int)soff, kStreamPolicy);
            if constexpr (GATED)
                wv[c] |= __builtin_amdgcn_raw_buffer_load_b128(wsrc2, (int)(w_voff2 + c * 64), (int)soff,
                                                               kStreamPolicy);
        }
#pragma unroll
        for (int c = 0; c < CHUNK; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xv[c][mt] = buf_load16(xsrc, x_voff[mt] + c * 64, soff);
        // With two token tiles the scheduler would interleave MFMAs (and
        // their waits) into the load block and cap the bytes in flight; with
        // one tile its interleave measured faster, so it is left alone.
        if (MT == 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < CHUNK; ++c)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, wv[c]),
                                                                   __builtin_bit_cast(bf16x8v, xv[c][mt]),
                                                                   acc[mt], 0, 0, 0);
    }

    // accumulator element v of token tile mt: weight row 4*(lane/16) + v,
    // token mt*16 + lane%16
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][(mt * 4 + v) * 64 + lane] = acc[mt][v];
    __syncthreads();

    for (int idx = t; idx < MT * 4 * 64; idx += KS * 64) gemv_store<EPI, MT, KS>(g, bt, n0, idx, red);
}

// Segmented stream (used whenever a wave's K range is a multiple of 128):
// every weight load instruction reads 4 rows x 256 contiguous bytes (lane l:
// row 4i + l/16, bytes 16*(l%16) of the segment); HBM serves that at ~6.5
// TB/s where the 16-rows-x-64-bytes pattern above reaches ~5.3 (pure-read
// measurements on MI355X).  Each wave moves a 4 KiB unit (16 rows x 128 k)
// through its own 4 KiB LDS slot into the 16x16x32 fragment order, with no
// workgroup barrier: the 16-byte slot is i*64 + a*16 + (b ^ (4i + a)) on the
// write (instruction i, lane (a, b)) and (r/4)*64 + (r%4)*16 + ((4s + g) ^ r)
// on the read (k-step s, lane (g, r)), conflict-free both ways.  A lane's
// fragment holds the same k values as in gemv_bf16_kernel, so for the same
// split of K the sums are formed in the same order.  D units (loads of
// weights and tokens) are kept in flight per wave.  With two token tiles
// (M > 16) the token rows are read the same way (a 16-token x 128-k unit is
// a weight unit's shape) and regrouped through the same slot after the
// weights: read straight into fragments, each token load touched 16
// half-used cache lines instead of 8 whole ones, and those line accesses
// bound the kernel at M = 32 (measured 17% faster).  Sixteen-wave blocks
// have no registers for the regroup and run with one token tile only.
template <int EPI, int MT, int KS, int D>
__global__ void __launch_bounds__(KS * 64) gemv_seg_kernel(GemvDev g)
{
    __shared__ u32x4 ulds[KS][256];
    __shared__ float red[KS][MT * 4 * 64];

    constexpr bool GATED = epi_gated(EPI);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // batch entry fastest: the T shards' blocks of the same weight rows run
    // side by side (see seg_grid)
    const int bt = blockIdx.x % g.batch;
    const int n0 = (blockIdx.x / g.batch) * (GATED ? 8 : 16);   // first output column
    const int Kw = g.K / KS;
    const int kbeg = w * Kw;
    const int units = Kw / 128;

    // gated: instructions 0, 1 read gate rows 0..7, instructions 2, 3 the
    // matching up rows, which become rows 8..15 of the block
    const __amdgpu_buffer_rsrc_t wsrc =
        make_rsrc(g.W[bt] + (int64_t)n0 * g.ldw, (uint32_t)((GATED ? 8 : 16) * g.ldw * 2));
    const __amdgpu_buffer_rsrc_t wsrc2 = make_rsrc((GATED ? g.W2[bt] : g.W[bt]) + (int64_t)n0 * g.ldw,
                                                   (uint32_t)((GATED ? 8 : 16) * g.ldw * 2));
    const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(g.X[bt], (uint32_t)((int64_t)g.M * g.ldx * 2));

    const int a = lane >> 4, b = lane & 15;
    uint32_t w_voff[4];
    int wslot[4], rslot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w_voff[i] = (uint32_t)(((4 * (GATED ? (i & 1) : i) + a) * g.ldw + kbeg) * 2 + b * 16);
        wslot[i] = i * 64 + a * 16 + (b ^ (4 * i + a));
        rslot[i] = (b >> 2) * 64 + (b & 3) * 16 + ((4 * i + a) ^ b);
    }
    // token rows: regrouped (instruction i reads tokens 16mt + 4i + a, 256
    // contiguous bytes each) or read straight into fragments (lane: token
    // 16mt + b, k-chunk a of the 32-wide k-step i)
    constexpr bool XR = MT == 2;
    static_assert(!(XR && KS > 8), "two token tiles run on at most eight waves");
    uint32_t x_voff[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        x_voff[mt] = XR ? (uint32_t)(((mt * 16 + a) * g.ldx + kbeg) * 2 + b * 16)
                        : (uint32_t)(((mt * 16 + b) * g.ldx + kbeg + 8 * a) * 2);
    const uint32_t x_istep = XR ? (uint32_t)(4 * g.ldx * 2) : 64u;

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{};

    u32x4 wv[D][4], xv[D][4][MT];
    auto issue = [&](int u, int d) __attribute__((always_inline)) {
        const int so = u * 256;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (GATED && i >= 2)
                wv[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wsrc2, (int)w_voff[i], so, kStreamPolicy);
            else
                wv[d][i] = __builtin_amdgcn_raw_buffer_load_b128(wsrc, (int)w_voff[i], so, kStreamPolicy);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xv[d][s][mt] = buf_load16(xsrc, x_voff[mt] + s * x_istep, (uint32_t)so);
    };
    auto step = [&](int u, int d) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ulds[w][wslot[i]] = wv[d][i];
        u32x4 f[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) f[s] = ulds[w][rslot[s]];
        if constexpr (XR) {
            // the slot is reused: a wave's LDS operations complete in order
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ulds[w][wslot[i]] = xv[d][i][mt];
#pragma unroll
                for (int s = 0; s < 4; ++s) xv[d][s][mt] = ulds[w][rslot[s]];
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, f[s]),
                                                                   __builtin_bit_cast(bf16x8v, xv[d][s][mt]),
                                                                   acc[mt], 0, 0, 0);
        if (u + D < units) issue(u + D, d);
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < units) issue(d, d);
    for (int u = 0; u < units; u += D) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (u + d < units) step(u + d, d);
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][(mt * 4 + v) * 64 + lane] = acc[mt][v];
    __syncthreads();

    for (int idx = t; idx < MT * 4 * 64; idx += KS * 64) gemv_store<EPI, MT, KS>(g, bt, n0, idx, red);
}

// One-dimensional grid with the batch entry (TP shard) varying fastest, so
// the blocks in flight at any moment read the same weight rows for every
// shard.  A shard's block of W2^T or W_o^T is a column block of the full
// matrix: its 16 rows are short pieces (8 KiB, 2 KiB) at a long row stride,
// and with the shards side by side the pieces in flight join into whole
// rows.  Measured on the 80-layer decode stack (whole TP group, M = 8):
// down-projection 92.9 -> 81.4 us, out-projection 31.3 -> 21.9 us per layer,
// with bitwise-equal results.
dim3 seg_grid(const GemvDev &g, int epi, int batch)
{
    return dim3((unsigned)(g.N / (epi_gated(epi) ? 8 : 16) * batch));
}

template <int EPI, int MT, int KS>
hipError_t launch_ks(const GemvDev &g, int batch, hipStream_t s)
{
    const dim3 grid((unsigned)(g.N / (epi_gated(EPI) ? 8 : 16)), (unsigned)batch);
    if ((g.K / KS) % 128 == 0) {
        hipLaunchKernelGGL((gemv_seg_kernel<EPI, MT, KS, 2>), seg_grid(g, EPI, batch), dim3(KS * 64), 0, s, g);
        return hipGetLastError();
    }
    const int steps = g.K / KS / 32;  // MFMA k-steps per wave
    if (steps % 8 == 0)
        hipLaunchKernelGGL((gemv_bf16_kernel<EPI, MT, KS, 8>), grid, dim3(KS * 64), 0, s, g);
    else
        hipLaunchKernelGGL((gemv_bf16_kernel<EPI, MT, KS, 2>), grid, dim3(KS * 64), 0, s, g);
    return hipGetLastError();
}

template <int EPI, int MT>
hipError_t launch_mt(const GemvDev &g, int batch, int num_cu, hipStream_t s)
{
    // Split K over the most waves (8 or 4) that still leaves each wave at
    // least 256 elements and an even number of 32-wide k-steps; K is a
    // multiple of 64, so a single wave always works.  Eight waves per block
    // with two blocks per CU streamed faster than sixteen with one.  A grid
    // with fewer blocks than CUs (a narrow projection such as one rank's
    // query, key or value block) has too few bytes in flight at eight
    // waves: it takes sixteen, each wave with two 4 KiB units in flight.
    // With two token tiles it stays at eight waves, where the token rows are
    // regrouped (sixteen waves have no registers for that); measured on one
    // rank's decode Q/K/V projection at M = 32: 16.4 against 22.3 us.
    if constexpr (MT == 1) {
        const int blocks = g.N / (epi_gated(EPI) ? 8 : 16) * batch;
        if (blocks < num_cu && (g.K / 16) % 128 == 0 && g.K / 16 >= 256) {
            hipLaunchKernelGGL((gemv_seg_kernel<EPI, MT, 16, 2>), seg_grid(g, EPI, batch), dim3(16 * 64), 0, s, g);
            return hipGetLastError();
        }
    }
    if (g.K % (8 * 64) == 0 && g.K / 8 >= 256) return launch_ks<EPI, MT, 8>(g, batch, s);
    if (g.K % (4 * 64) == 0 && g.K / 4 >= 256) return launch_ks<EPI, MT, 4>(g, batch, s);
    return launch_ks<EPI, MT, 1>(g, batch, s);
}

}  // namespace

hipError_t launch_gemv_bf16(const GemmArgs &a, Epilogue epi, int num_cu, hipStream_t s)
{
    GemvDev g;
    for (int b = 0; b < kMaxBatch; ++b) {
        const int src = b < a.batch ? b : 0;
        g.X[b] = static_cast<const __bf16 *>(a.A[src]);
        g.W[b] = static_cast<const __bf16 *>(a.B[src]);
        g.bias[b] = static_cast<const __bf16 *>(a.bias[src]);
        g.W2[b] = static_cast<const __bf16 *>(a.B2[src]);
        g.bias2[b] = static_cast<const __bf16 *>(a.bias2[src]);
        g.C[b] = a.C[src];
    }
    g.ldx = a.lda;
    g.ldw = a.ldb;
    for (int b = 0; b < kMaxBatch; ++b) g.ldc[b] = ldc_of(a, b < a.batch ? b : 0);
    g.M = (int)a.M;
    g.N = (int)a.N;
    g.K = (int)a.K;
    g.batch = a.batch;
    const bool two = a.M > 16;
    switch (epi) {
    case EPI_BIAS_GELU:
        return two ? launch_mt<EPI_BIAS_GELU, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_BIAS_GELU, 1>(g, a.batch, num_cu, s);
    case EPI_STORE_F32:
        return two ? launch_mt<EPI_STORE_F32, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_STORE_F32, 1>(g, a.batch, num_cu, s);
    case EPI_BIAS_GELU_ERF:
        return two ? launch_mt<EPI_BIAS_GELU_ERF, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_BIAS_GELU_ERF, 1>(g, a.batch, num_cu, s);
    case EPI_GATED_TANH:
        return two ? launch_mt<EPI_GATED_TANH, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_GATED_TANH, 1>(g, a.batch, num_cu, s);
    case EPI_GATED_ERF:
        return two ? launch_mt<EPI_GATED_ERF, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_GATED_ERF, 1>(g, a.batch, num_cu, s);
    case EPI_BIAS:
        return two ? launch_mt<EPI_BIAS, 2>(g, a.batch, num_cu, s) : launch_mt<EPI_BIAS, 1>(g, a.batch, num_cu, s);
    default:   // the gradient epilogues run on the MFMA GEMM only
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
