// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by abi.cpp: shapes in
// range, K a multiple of 64, N a multiple of 64, 16-byte aligned pointers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tpk {

// What a GEMM does with its fp32 accumulator tile.
enum Epilogue : int {
    EPI_BIAS_GELU = 0,  // + bias[n] (if any), GeLU(tanh), store in the input dtype
    EPI_STORE_F32 = 1,  // store the fp32 accumulator (row-parallel partial)
};

// C[m][n] = sum_k A[m][k] * B[n][k]  (both operands K-contiguous), then the
// epilogue.  A: M rows, stride lda; B: N rows, stride ldb; C: stride ldc.
// `batch` independent problems of the same shape (one per TP shard when the
// whole TP group is emulated on one GPU) may be launched together; entry b
// of each pointer array belongs to problem b.
constexpr int kMaxBatch = 8;
struct GemmArgs {
    const void *A[kMaxBatch];
    int64_t lda;
    const void *B[kMaxBatch];
    int64_t ldb;
    const void *bias[kMaxBatch];  // [N] or nullptr (EPI_BIAS_GELU only)
    void *C[kMaxBatch];
    int64_t ldc;
    int64_t M, N, K;
    int batch;
};

// bf16 x bf16 -> fp32 accumulate, MFMA tiles; for M > 32.
hipError_t launch_gemm_bf16(const GemmArgs &g, Epilogue epi, int num_cu, hipStream_t s);
// bf16 skinny-M (M <= 32) weight-streaming path.
hipError_t launch_gemv_bf16(const GemmArgs &g, Epilogue epi, int num_cu, hipStream_t s);
// fp32 x fp32 -> fp32, exact fp32 FMA (no reduced-precision tricks).
hipError_t launch_gemm_f32(const GemmArgs &g, Epilogue epi, hipStream_t s);

// out = (residual ? residual : 0) + sum_j partials[j]; optional bf16 copy,
// optionally row-RMS-normalised.
constexpr int kMaxPartials = 8;
hipError_t launch_shard_reduce(const float *const *partials, int T, const float *residual,
                               float *out, void *out_bf16, int64_t M, int64_t H, bool rms,
                               float eps, hipStream_t s);

}  // namespace tpk
