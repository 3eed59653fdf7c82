// Sum of the T row-parallel partials (the on-device stand-in for the
// All-Reduce-Sum), with the optional residual add and bf16 copy:
//   s = P_0 + P_1 + ... + P_{T-1}   (fixed order, fp32)
//   out = residual ? residual + s : s
//   out_bf16 = bf16(out)  or  bf16(out / sqrt(mean_row(out^2) + eps))
// Pure streaming: (T + 1 [+1]) * 4 bytes read and 4 [+2] written per element,
// so it is HBM-bound.  Every lane moves 16 bytes per tensor per step, and all
// T loads of a step are issued before the adds.  The row-normalised variant
// runs one workgroup per row and reduces the sum of squares with wavefront
// shuffles, then across the sixteen waves through LDS.
// Partials larger than half the 256 MB last-level cache are read with
// non-temporal loads: they cannot stay cached anyway, and at the 80-layer
// stack's prefill shape (eight 128 MiB partials and the residual, in place)
// the plain reduce took 221 instead of 258 us with them (6.1 against 5.2
// TB/s); partials the cache does hold (the 2048-token block's four) are
// read faster through it.
#include "device_common.h"
#include "tp_kernels.h"

namespace tpk {
namespace {

struct PartialPtrs {
    const f32x4 *p[kMaxPartials];
};

__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 v)
{
    const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    return __builtin_bit_cast(u32x2, b);
}

template <bool STREAM>
__device__ __forceinline__ f32x4 load_part(const f32x4 *p)
{
    if constexpr (STREAM)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int T, bool STREAM>
__device__ __forceinline__ f32x4 sum_partials(const PartialPtrs &P, int64_t i)
{
    f32x4 v[T];
#pragma unroll
    for (int j = 0; j < T; ++j) v[j] = load_part<STREAM>(P.p[j] + i);
    f32x4 s = v[0];
#pragma unroll
    for (int j = 1; j < T; ++j) s += v[j];
    return s;
}

template <int T, bool STREAM>
__global__ void __launch_bounds__(256) reduce_kernel(PartialPtrs P, const f32x4 *residual, f32x4 *out,
                                                     u32x2 *out_bf16, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        f32x4 s = sum_partials<T, STREAM>(P, i);
        if (residual) s = residual[i] + s;
        out[i] = s;
        if (out_bf16) out_bf16[i] = pack_bf16x4(s);
    }
}

// Row-normalised variant: one workgroup of RMS_THREADS threads per row.  Each
// pass of a thread covers two 16-byte elements of every tensor, and all
// 2(T [+1]) loads of a pass are issued before the adds, so a workgroup keeps
// a whole H = 8192 row (8 partials + residual, 288 KiB) in flight at once:
// at decode sizes a handful of rows is the whole launch, and its time is the
// latency of one round of loads (80-layer decode stack at M = 8: 9.3 us with
// 256 threads and one element per pass, 5.9 us like this).
constexpr int RMS_THREADS = 1024;

template <int T, bool STREAM>
__global__ void __launch_bounds__(RMS_THREADS) reduce_rms_kernel(PartialPtrs P, const f32x4 *residual, f32x4 *out,
                                                                 u32x2 *out_bf16, int64_t h4, float inv_h, float eps)
{
    constexpr int NT = RMS_THREADS, NWV = NT / 64;
    __shared__ float wsum[NWV];
    const int64_t base = (int64_t)blockIdx.x * h4;
    float ss = 0.0f;
    f32x4 keep[2] = {};   // a row of one pass keeps its sums here for the bf16 copy
    for (int64_t c = threadIdx.x; c < h4; c += 2 * NT) {
        // the second element of a pass past the row end re-reads the last
        // element of the row and is not stored
        const int64_t c2 = c + NT < h4 ? c + NT : h4 - 1;
        f32x4 v[2][T + 1];
#pragma unroll
        for (int j = 0; j < T; ++j) {
            v[0][j] = load_part<STREAM>(P.p[j] + base + c);
            v[1][j] = load_part<STREAM>(P.p[j] + base + c2);
        }
        if (residual) {
            v[0][T] = residual[base + c];
            v[1][T] = residual[base + c2];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (e == 1 && c + NT >= h4) break;
            f32x4 s = v[e][0];
#pragma unroll
            for (int j = 1; j < T; ++j) s += v[e][j];
            if (residual) s = v[e][T] + s;
            out[base + (e ? c2 : c)] = s;
            keep[e] = s;
            ss += s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3];
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) tot += wsum[w];
    const float r = rsqrtf(tot * inv_h + eps);
    if (h4 <= 2 * NT) {   // one pass (H <= 8192): the sums are still in registers
        const int64_t c = threadIdx.x;
        if (c < h4) out_bf16[base + c] = pack_bf16x4(keep[0] * r);
        if (c + NT < h4) out_bf16[base + c + NT] = pack_bf16x4(keep[1] * r);
        return;
    }
    // each thread re-reads only the elements it wrote itself
    for (int64_t c = threadIdx.x; c < h4; c += NT) out_bf16[base + c] = pack_bf16x4(out[base + c] * r);
}

template <int T>
hipError_t launch_t(const PartialPtrs &P, const float *residual, float *out, void *ob, int64_t M,
                    int64_t H, bool rms, float eps, hipStream_t s)
{
    const f32x4 *r4 = reinterpret_cast<const f32x4 *>(residual);
    f32x4 *o4 = reinterpret_cast<f32x4 *>(out);
    u32x2 *b4 = static_cast<u32x2 *>(ob);
    const bool stream = (int64_t)T * M * H * 4 > (int64_t(128) << 20);
    if (rms) {
        const dim3 grid((unsigned)M), block(RMS_THREADS);
        if (stream)
            hipLaunchKernelGGL((reduce_rms_kernel<T, true>), grid, block, 0, s, P, r4, o4, b4, H / 4, 1.0f / (float)H,
                               eps);
        else
            hipLaunchKernelGGL((reduce_rms_kernel<T, false>), grid, block, 0, s, P, r4, o4, b4, H / 4, 1.0f / (float)H,
                               eps);
    } else {
        const int64_t n4 = M * H / 4;
        const dim3 grid((unsigned)std::min<int64_t>((n4 + 255) / 256, 1 << 16)), block(256);
        if (stream)
            hipLaunchKernelGGL((reduce_kernel<T, true>), grid, block, 0, s, P, r4, o4, b4, n4);
        else
            hipLaunchKernelGGL((reduce_kernel<T, false>), grid, block, 0, s, P, r4, o4, b4, n4);
    }
    return hipGetLastError();
}

// Column sums of bf16 matrices X_j [M][N] (row stride ld), j < batch, into
// fp32 out_j[N], in a fixed order.  A workgroup owns 64 columns of one matrix,
// so every row it reads is one whole 128-byte line: thread t reads 8 columns
// (16 bytes) from rows t/8, t/8 + 64, t/8 + 128, ... with four loads in flight.
// The 64 row lanes' sums are then added through LDS, eight lanes at a time
// and the eight group sums in group order.  blockIdx.y picks the matrix, so
// the T shards of a group fill the chip in one launch.
struct ColsumPtrs {
    const __bf16 *x[kMaxPartials];
    float *out[kMaxPartials];
};

__global__ void __launch_bounds__(512) colsum_kernel(ColsumPtrs P, int64_t ld, int M, int N, int accumulate)
{
    constexpr int RL = 64;   // row lanes
    __shared__ float part[RL][65];
    __shared__ float part2[8][64];
    const int t = threadIdx.x, cc = t & 7, rl = t >> 3;
    const int n0 = blockIdx.x * 64 + 8 * cc;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    auto add = [&](u32x4 w) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __builtin_bit_cast(float, w[i] << 16);
            acc[2 * i + 1] += __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        }
    };
    if (n0 < N) {
        const __bf16 *col = P.x[blockIdx.y] + n0;
        int m = rl;
        for (; m + 3 * RL < M; m += 4 * RL) {
            u32x4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = *reinterpret_cast<const u32x4 *>(col + (int64_t)(m + RL * u) * ld);
#pragma unroll
            for (int u = 0; u < 4; ++u) add(w[u]);
        }
        for (; m < M; m += RL) add(*reinterpret_cast<const u32x4 *>(col + (int64_t)m * ld));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rl][8 * cc + e] = acc[e];
    __syncthreads();
    {
        const int c = t & 63, grp = t >> 6;   // 8 groups x 64 columns = 512 threads
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) sum += part[8 * grp + r][c];
        part2[grp][c] = sum;
    }
    __syncthreads();
    if (t < 64) {
        const int n = blockIdx.x * 64 + t;
        float sum = 0.0f;
#pragma unroll
        for (int g = 0; g < 8; ++g) sum += part2[g][t];
        float *out = P.out[blockIdx.y];
        if (n < N) out[n] = accumulate ? out[n] + sum : sum;
    }
}

}  // namespace

hipError_t launch_colsum_bf16(const void *const *X, int batch, int64_t ld, int64_t M, int64_t N,
                              float *const *out, bool accumulate, hipStream_t s)
{
    if (batch < 1 || batch > kMaxPartials) return hipErrorInvalidValue;
    ColsumPtrs P{};
    for (int j = 0; j < batch; ++j) {
        P.x[j] = static_cast<const __bf16 *>(X[j]);
        P.out[j] = out[j];
    }
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)batch);
    hipLaunchKernelGGL(colsum_kernel, grid, dim3(512), 0, s, P, ld, (int)M, (int)N, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_shard_reduce(const float *const *partials, int T, const float *residual, float *out,
                               void *out_bf16, int64_t M, int64_t H, bool rms, float eps, hipStream_t s)
{
    PartialPtrs P{};
    for (int j = 0; j < T; ++j) P.p[j] = reinterpret_cast<const f32x4 *>(partials[j]);
    switch (T) {
    case 1: return launch_t<1>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 2: return launch_t<2>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 3: return launch_t<3>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 4: return launch_t<4>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 5: return launch_t<5>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 6: return launch_t<6>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 7: return launch_t<7>(P, residual, out, out_bf16, M, H, rms, eps, s);
    case 8: return launch_t<8>(P, residual, out, out_bf16, M, H, rms, eps, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace tpk
