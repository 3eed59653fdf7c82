// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by abi.cpp: shapes in
// range, K a multiple of 64, N a multiple of 64, 16-byte aligned pointers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tpk {

// What a GEMM does with its fp32 accumulator tile.
enum Epilogue : int {
    EPI_BIAS_GELU = 0,      // + bias[n] (if any), GeLU (tanh form), store in the input dtype
    EPI_STORE_F32 = 1,      // store the fp32 accumulator (row-parallel partial)
    EPI_BIAS_GELU_ERF = 2,  // + bias[n] (if any), GeLU (exact x*Phi(x)), input dtype
    EPI_GATED_TANH = 3,     // GeLU_tanh(gate + bias[n]) * (up + bias2[n]), input dtype
    EPI_GATED_ERF = 4,      // GeLU_erf(gate + bias[n]) * (up + bias2[n]), input dtype
    EPI_BIAS = 5,           // + bias[n] (if any), no activation, input dtype
    EPI_GELU_GRAD_TANH = 6, // acc * g'(aux[m][n]) (tanh-form GeLU derivative), bf16
    EPI_GELU_GRAD_ERF = 7,  // acc * g'(aux[m][n]) (exact GeLU derivative), bf16
    EPI_ACC_F32 = 8,        // C[m][n] += acc, fp32
};
constexpr bool epi_gated(int e) { return e == EPI_GATED_TANH || e == EPI_GATED_ERF; }
constexpr bool epi_act_grad(int e) { return e == EPI_GELU_GRAD_TANH || e == EPI_GELU_GRAD_ERF; }
constexpr bool epi_has_bias(int e) { return e == EPI_BIAS_GELU || e == EPI_BIAS_GELU_ERF || e == EPI_BIAS; }

// Operand layouts of the bf16 MFMA GEMM (K-major: element (r, k) at k*ld + r).
enum Layout : int {
    LAYOUT_KCONTIG = 0,    // A [M][K], B [N][K]
    LAYOUT_B_KMAJOR = 1,   // A [M][K], B stored [K][N]
    LAYOUT_AB_KMAJOR = 2,  // A stored [K][M], B stored [K][N]
};

// C[m][n] = sum_k A[m][k] * B[n][k]  (both operands K-contiguous), then the
// epilogue.  A: M rows, stride lda; B: N rows, stride ldb; C: stride ldc.
// `batch` independent problems of the same shape (one per TP shard when the
// whole TP group is emulated on one GPU) may be launched together; entry b
// of each pointer array belongs to problem b.  The gated epilogues take a
// second weight matrix B2 (the up rows; B holds the gate rows, same N, K and
// stride) and a second bias, and write N columns.
constexpr int kMaxBatch = 8;
struct GemmArgs {
    const void *A[kMaxBatch];
    int64_t lda;
    const void *B[kMaxBatch];
    int64_t ldb;
    const void *bias[kMaxBatch];   // [N] or nullptr (activation epilogues)
    const void *B2[kMaxBatch];     // gated epilogues: up rows, else unused
    const void *bias2[kMaxBatch];  // gated epilogues: up bias [N] or nullptr
    void *C[kMaxBatch];
    int64_t ldc;
    int64_t ldc_b[kMaxBatch];      // per-problem row stride of C; 0 = ldc
    void *aux[kMaxBatch];          // [M][N] bf16, stride ldaux: the GeLU input, written by the
    int64_t ldaux;                 //   GeLU epilogues when set, read by the gradient epilogues
    int64_t M, N, K;
    int batch;
    int layout;                    // Layout (bf16 MFMA GEMM only)
};
inline int64_t ldc_of(const GemmArgs &g, int b) { return g.ldc_b[b] ? g.ldc_b[b] : g.ldc; }

// bf16 x bf16 -> fp32 accumulate, MFMA tiles; for M > 32.
hipError_t launch_gemm_bf16(const GemmArgs &g, Epilogue epi, int num_cu, hipStream_t s);
// bf16 skinny-M (M <= 32) weight-streaming path.
hipError_t launch_gemv_bf16(const GemmArgs &g, Epilogue epi, int num_cu, hipStream_t s);
// fp32 x fp32 -> fp32, exact fp32 FMA (no reduced-precision tricks).
hipError_t launch_gemm_f32(const GemmArgs &g, Epilogue epi, hipStream_t s);

// Scaled dot-product attention of one rank's heads, head dim 128, bf16:
// Q rows b*Sq + s (stride ldq), K/V rows b*Lk + t (strides ldk, ldv), ctx
// rows like Q (stride ldo); query head h at columns 128h, key/value head g
// at columns 128g; query head h reads key/value head h / (nh / nkv).
struct AttnArgs {
    const void *Q, *K, *V;
    void *O;
    const int32_t *kv_len;   // device [Bs] valid keys per sequence, or nullptr (Lk)
    int64_t ldq, ldk, ldv, ldo;
    int64_t Bs, Sq, Lk;
    int nh, nkv;
    bool causal;
    void *ws;                // decode partials (AttnPlan::ws_bytes), else unused
};
// Which kernel runs and, for the split-key decode kernel, how the keys are
// split and how much workspace the partials take.  Depends on shapes only.
struct AttnPlan {
    bool decode;
    int nsplit, chunk;
    size_t ws_bytes;
    size_t partials_offset;   // the workspace: arrival counters at 0, the partials from here
};
AttnPlan attn_plan(int64_t Bs, int64_t Sq, int64_t Lk, int nh, int nkv);
constexpr int kAttnD = 128;             // head dim
constexpr int kAttnDecRows = 8;         // most query rows per key/value head on the decode kernel
constexpr int kAttnDecMaxChunk = 512;   // most keys per decode workgroup
constexpr int kAttnMaxSplit = 4096;     // most key chunks per sequence on the decode path
constexpr int kAttnMaxArrivals = 4096;  // most (sequence, key/value head) pairs on the decode path
hipError_t launch_attn_bf16(const AttnArgs &a, int num_cu, hipStream_t s);


// out = (residual ? residual : 0) + sum_j partials[j]; optional bf16 copy,
// optionally row-RMS-normalised.
constexpr int kMaxPartials = 8;

// out_j[n] (+)= sum_m X_j[m][n] for bf16 X_j [M][N], j < batch <= kMaxPartials
// (row stride ld, N and ld multiples of 8), fp32, in a fixed order; one launch.
hipError_t launch_colsum_bf16(const void *const *X, int batch, int64_t ld, int64_t M, int64_t N,
                              float *const *out, bool accumulate, hipStream_t s);
hipError_t launch_shard_reduce(const float *const *partials, int T, const float *residual,
                               float *out, void *out_bf16, int64_t M, int64_t H, bool rms,
                               float eps, hipStream_t s);

// Staging area of tp_mlp_shard_fwd_noalloc: a file-scope device array of
// kScratchBytes per GPU (scratch.hip).  scratch_base gives this device's
// copy's address (looked up once per device, the device current).
constexpr int64_t kScratchBytes = int64_t(16) << 20;
hipError_t scratch_base(void **out);

}  // namespace tpk
