// Test double of the kernel launchers (csrc/tp_kernels.h) and of the three
// HIP runtime calls the C ABI makes, for a CPU-only build of abi.cpp and
// plan.cpp with AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing
// here touches a GPU: each launch is appended to a log (what the ABI would
// have enqueued, with its shape), and the log is read back through the
// rec_* functions.  The launchers also check the invariants tp_kernels.h
// states for their arguments and count every violation.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "tp_kernels.h"

namespace {

enum Kind { K_GEMM_BF16 = 0, K_GEMV_BF16 = 1, K_GEMM_F32 = 2, K_ATTN = 3, K_COLSUM = 4, K_REDUCE = 5 };

struct Rec {
    int64_t v[8];   // kind, epilogue or flags, M, N, K, batch or T, layout or rms, variant
};

std::mutex g_mu;
std::vector<Rec> g_log;
int64_t g_violations = 0;

bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void push(Rec r)
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_log.push_back(r);
}

void violation()
{
    std::lock_guard<std::mutex> lk(g_mu);
    ++g_violations;
}

hipError_t gemm(int kind, const tpk::GemmArgs &g, tpk::Epilogue epi)
{
    if (g.batch < 1 || g.batch > tpk::kMaxBatch || g.M < 1 || g.N < 1 || g.K < 1) violation();
    for (int b = 0; b < g.batch && b < tpk::kMaxBatch; ++b)
        if (!g.A[b] || !g.B[b] || !g.C[b] || !al16(g.A[b]) || !al16(g.B[b]) || !al16(g.C[b])) violation();
    if (kind != K_GEMM_F32 && g.layout == tpk::LAYOUT_KCONTIG && g.K % 64 != 0) violation();
    push(Rec{{kind, (int64_t)epi, g.M, g.N, g.K, g.batch, g.layout, 0}});
    return hipSuccess;
}

}  // namespace

namespace tpk {

hipError_t launch_gemm_bf16(const GemmArgs &g, Epilogue epi, int, hipStream_t) { return gemm(K_GEMM_BF16, g, epi); }
hipError_t launch_gemv_bf16(const GemmArgs &g, Epilogue epi, int, hipStream_t)
{
    if (g.M > 32) violation();
    return gemm(K_GEMV_BF16, g, epi);
}
hipError_t launch_gemm_f32(const GemmArgs &g, Epilogue epi, hipStream_t) { return gemm(K_GEMM_F32, g, epi); }

hipError_t launch_attn_bf16(const AttnArgs &a, int, hipStream_t)
{
    const AttnPlan p = attn_plan(a.Bs, a.Sq, a.Lk, a.nh, a.nkv);
    if (p.decode && p.ws_bytes > 0 && !a.ws) violation();
    push(Rec{{K_ATTN, a.causal ? 1 : 0, a.Bs * a.Sq, a.nh, a.Lk, a.Bs, p.decode ? 1 : 0, p.nsplit}});
    return hipSuccess;
}

hipError_t launch_colsum_bf16(const void *const *X, int batch, int64_t ld, int64_t M, int64_t N, float *const *out,
                              bool accumulate, hipStream_t)
{
    if (batch < 1 || batch > kMaxPartials || N % 8 != 0 || ld % 8 != 0) violation();
    for (int b = 0; b < batch && b < kMaxPartials; ++b)
        if (!X[b] || !out[b]) violation();
    push(Rec{{K_COLSUM, accumulate ? 1 : 0, M, N, 0, batch, 0, 0}});
    return hipSuccess;
}

hipError_t launch_shard_reduce(const float *const *partials, int T, const float *residual, float *out, void *out_bf16,
                               int64_t M, int64_t H, bool rms, float, hipStream_t)
{
    if (T < 1 || T > kMaxPartials || !out || (rms && !out_bf16)) violation();
    for (int j = 0; j < T && j < kMaxPartials; ++j)
        if (!partials[j] || !al16(partials[j])) violation();
    push(Rec{{K_REDUCE, (residual ? 1 : 0) | (out_bf16 ? 2 : 0), M, H, 0, T, rms ? 1 : 0, 0}});
    return hipSuccess;
}

// the staging buffer of tp_mlp_shard_fwd_noalloc: a fake, 256-byte aligned address
hipError_t scratch_base(void **out)
{
    *out = reinterpret_cast<void *>(uintptr_t(0xABC) << 32);
    return hipSuccess;
}

}  // namespace tpk

// The HIP runtime calls of abi.cpp: one device with 256 compute units.
extern "C" {

hipError_t hipGetDevice(int *dev)
{
    *dev = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int)
{
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t) { return "recorded launch (no GPU)"; }

// log access for the tests
void rec_reset()
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_log.clear();
    g_violations = 0;
}

int64_t rec_count()
{
    std::lock_guard<std::mutex> lk(g_mu);
    return (int64_t)g_log.size();
}

int64_t rec_violations()
{
    std::lock_guard<std::mutex> lk(g_mu);
    return g_violations;
}

// copies entry k's eight fields into out; returns 0, or -1 past the end
int rec_get(int64_t k, int64_t *out)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (k < 0 || k >= (int64_t)g_log.size()) return -1;
    for (int f = 0; f < 8; ++f) out[f] = g_log[(size_t)k].v[f];
    return 0;
}

}  // extern "C"
