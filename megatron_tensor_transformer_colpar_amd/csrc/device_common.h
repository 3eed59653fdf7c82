// Device helpers shared by the HIP kernels: vector types, buffer resources,
// the GeLU epilogue and the workgroup -> tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_kernels.h"

namespace tpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over [base, base + bytes): loads at or past the end return
// zero, which makes ragged tiles free.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// GeLU, tanh form (Hendrycks & Gimpel, arXiv:1606.08415):
//   g(x) = x/2 * (1 + tanh(u)),  u = sqrt(2/pi) * (x + 0.044715 x^3).
// Evaluated through (1 + tanh u)/2 = 1/(1 + e^(-2u)) = 1/(1 + 2^z) with
// z = x (c1 + c2 x^2), c1 = -2 sqrt(2/pi) log2(e), c2 = 0.044715 c1: a
// square, one fma and one multiply, the hardware exp2 and reciprocal, an add
// and a multiply (two fewer vector instructions per element than forming u
// and exp(-2u); this epilogue is bound by them).  The limits are right:
// x -> -inf gives 2^z -> inf and g -> -0; x -> +inf gives g -> x.
__device__ __forceinline__ float gelu_tanh(float x)
{
    constexpr float c1 = -2.302208198144325f;    // -2 sqrt(2/pi) log2(e)
    constexpr float c2 = -0.1029432395800235f;   // 0.044715 * c1
    const float e = __builtin_amdgcn_exp2f(x * fmaf(c2, x * x, c1));
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// GeLU, exact form (Hendrycks & Gimpel): g(x) = x * Phi(x)
//   = x/2 * (1 + erf(x / sqrt 2)), erf from the device library.
__device__ __forceinline__ float gelu_erf(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// GeLU derivatives ([GELU]).  Tanh form: with s = (1 + tanh v)/2 =
// 1/(1 + e^(-2v)), v = c(x + a x^3), g'(x) = s + 2 x s (1 - s) c (1 + 3 a x^2).
// Exact form: g'(x) = Phi(x) + x phi(x).
__device__ __forceinline__ float gelu_tanh_grad(float x)
{
    constexpr float c = 0.7978845608028654f, a = 0.044715f;
    const float s = __fdividef(1.0f, 1.0f + __expf(-2.0f * c * x * (1.0f + a * x * x)));
    return s + 2.0f * x * s * (1.0f - s) * c * (1.0f + 3.0f * a * x * x);
}
__device__ __forceinline__ float gelu_erf_grad(float x)
{
    return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.3989422804014327f * __expf(-0.5f * x * x);
}

template <int EPI>
__device__ __forceinline__ float act_grad(float x)
{
    if constexpr (EPI == EPI_GELU_GRAD_ERF)
        return gelu_erf_grad(x);
    else
        return gelu_tanh_grad(x);
}

// The activation an epilogue applies.
template <int EPI>
__device__ __forceinline__ float act(float x)
{
    if constexpr (EPI == EPI_BIAS)
        return x;
    else if constexpr (EPI == EPI_BIAS_GELU_ERF || EPI == EPI_GATED_ERF)
        return gelu_erf(x);
    else
        return gelu_tanh(x);
}

// Workgroup id -> (batch entry, tile_m, tile_n).  Consecutive workgroup ids
// are dealt round-robin to the 8 XCDs, each with its own L2; this remap gives
// every XCD a contiguous run of logical tiles, and walks the logical tiles of
// one batch entry in groups of GROUP_M tile-rows so the tiles in flight on
// one XCD share A and B panels.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int bid, int batch, int tiles_m, int tiles_n, int &bt, int &tm,
                                         int &tn)
{
    const int per_batch = tiles_m * tiles_n;
    const int total = batch * per_batch;
    int logical = bid;
    if ((total & 7) == 0) {
        const int per_xcd = total >> 3;
        logical = (bid & 7) * per_xcd + (bid >> 3);
    }
    bt = logical / per_batch;
    logical -= bt * per_batch;
    const int per_group = GROUP_M * tiles_n;
    const int group = logical / per_group;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int r = logical - group * per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

// Workgroup id -> (batch entry, tile_m, tile_n) for problems whose tile
// columns split evenly over the 8 XCDs: XCD x owns columns [x W, (x+1) W)
// of every batch entry, W = tiles_n / 8, and walks them entry by entry in
// groups of 8 tile rows.  Each round of an XCD's workgroups still covers an
// 8 x W block (the L2 reuse of map_tile), but every XCD works on the same
// entry at a time and keeps its B panels from round to round: the first
// round of an entry touches each of its B panels once and the later rounds
// find them in the last-level cache, instead of fetching new panels from
// HBM at every tile start.
__device__ __forceinline__ void map_tile_bands(int bid, int tiles_m, int tiles_n, int &bt, int &tm, int &tn)
{
    const int x = bid & 7, W = tiles_n >> 3, per_entry = tiles_m * W;
    int l = bid >> 3;
    bt = l / per_entry;
    l -= bt * per_entry;
    const int group = l / (8 * W), r = l - group * 8 * W;
    const int first_m = group * 8;
    const int gsize = min(tiles_m - first_m, 8);
    tm = first_m + r % gsize;
    tn = x * W + r / gsize;
}

}  // namespace tpk
