// fp32 GEMM, exact fp32 FMA on the vector ALUs (no bf16 or tf32-style
// splitting), for the fp32 precision mode:
//   C[m][n] = sum_k A[m][k] * B[n][k], then bias + GeLU (either form), a
//   plain store, or, gated, GeLU(gate + bias) * (up + bias2) with the up
//   product taken against a second matrix B2 in the same pass.
// A 64x64 output tile per 256-thread workgroup, 4x4 outputs per thread, K in
// 16-wide slices through LDS (stored k-major so a thread's 4 rows / 4 columns
// are one 16-byte read each).  Rows past M or N are read as zero.
#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

constexpr int TB = 64, TK = 16;

struct GemmF32Dev {
    const float *A;
    const float *B;
    const float *bias;
    const float *B2;      // gated: up rows
    const float *bias2;   // gated: up bias
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_n;
};

template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmF32Dev g)
{
    constexpr bool GATED = epi_gated(EPI);
    __shared__ f32x4 As[TK][TB / 4];
    __shared__ f32x4 Bs[TK][TB / 4];
    __shared__ f32x4 B2s[GATED ? TK : 1][TB / 4];

    const int t = threadIdx.x;
    const int m0 = (blockIdx.x / g.tiles_n) * TB, n0 = (blockIdx.x % g.tiles_n) * TB;
    const int tx = t & 15, ty = t >> 4;

    const __amdgpu_buffer_rsrc_t asrc =
        make_rsrc(g.A + (int64_t)m0 * g.lda, (uint32_t)((int64_t)min(TB, g.M - m0) * g.lda * 4));
    const __amdgpu_buffer_rsrc_t bsrc =
        make_rsrc(g.B + (int64_t)n0 * g.ldb, (uint32_t)((int64_t)min(TB, g.N - n0) * g.ldb * 4));
    const __amdgpu_buffer_rsrc_t b2src =
        GATED ? make_rsrc(g.B2 + (int64_t)n0 * g.ldb, (uint32_t)((int64_t)min(TB, g.N - n0) * g.ldb * 4)) : bsrc;
    // loader: thread t reads 4 consecutive k of row t/4
    const int lr = t >> 2, lk = (t & 3) * 4;
    const uint32_t a_off = (uint32_t)((lr * g.lda + lk) * 4);
    const uint32_t b_off = (uint32_t)((lr * g.ldb + lk) * 4);

    float acc[4][4] = {}, acc2[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += TK) {
        const f32x4 av = __builtin_bit_cast(f32x4, buf_load16(asrc, a_off, (uint32_t)k0 * 4));
        const f32x4 bv = __builtin_bit_cast(f32x4, buf_load16(bsrc, b_off, (uint32_t)k0 * 4));
        float *as = reinterpret_cast<float *>(As);
        float *bs = reinterpret_cast<float *>(Bs);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            as[(lk + j) * TB + lr] = av[j];
            bs[(lk + j) * TB + lr] = bv[j];
        }
        if constexpr (GATED) {
            const f32x4 b2v = __builtin_bit_cast(f32x4, buf_load16(b2src, b_off, (uint32_t)k0 * 4));
            float *b2s = reinterpret_cast<float *>(B2s);
#pragma unroll
            for (int j = 0; j < 4; ++j) b2s[(lk + j) * TB + lr] = b2v[j];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TK; ++k) {
            const f32x4 a = As[k][ty];
            const f32x4 b = Bs[k][tx];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
            if constexpr (GATED) {
                const f32x4 b2 = B2s[k][tx];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc2[i][j] = __builtin_fmaf(a[i], b2[j], acc2[i][j]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= g.N) continue;
            float x = acc[i][j];
            if constexpr (GATED) {
                const float up = g.bias2 ? acc2[i][j] + g.bias2[n] : acc2[i][j];
                x = act<EPI>(g.bias ? x + g.bias[n] : x) * up;
            } else if (EPI != EPI_STORE_F32) {
                x = act<EPI>(g.bias ? x + g.bias[n] : x);
            }
            g.C[(int64_t)m * g.ldc + n] = x;
        }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, Epilogue epi, hipStream_t s)
{
    for (int b = 0; b < a.batch; ++b) {
        GemmF32Dev g;
        g.A = static_cast<const float *>(a.A[b]);
        g.B = static_cast<const float *>(a.B[b]);
        g.bias = static_cast<const float *>(a.bias[b]);
        g.B2 = static_cast<const float *>(a.B2[b]);
        g.bias2 = static_cast<const float *>(a.bias2[b]);
        g.C = static_cast<float *>(a.C[b]);
        g.lda = a.lda;
        g.ldb = a.ldb;
        g.ldc = ldc_of(a, b);
        g.M = (int)a.M;
        g.N = (int)a.N;
        g.K = (int)a.K;
        g.tiles_n = (int)((a.N + TB - 1) / TB);
        const dim3 grid((unsigned)(g.tiles_n * ((a.M + TB - 1) / TB)));
        switch (epi) {
        case EPI_BIAS_GELU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS_GELU>, grid, dim3(256), 0, s, g); break;
        case EPI_STORE_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE_F32>, grid, dim3(256), 0, s, g); break;
        case EPI_BIAS_GELU_ERF:
            hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS_GELU_ERF>, grid, dim3(256), 0, s, g);
            break;
        case EPI_GATED_TANH: hipLaunchKernelGGL(gemm_f32_kernel<EPI_GATED_TANH>, grid, dim3(256), 0, s, g); break;
        case EPI_GATED_ERF: hipLaunchKernelGGL(gemm_f32_kernel<EPI_GATED_ERF>, grid, dim3(256), 0, s, g); break;
        case EPI_BIAS: hipLaunchKernelGGL(gemm_f32_kernel<EPI_BIAS>, grid, dim3(256), 0, s, g); break;
        default: return hipErrorInvalidValue;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tpk
