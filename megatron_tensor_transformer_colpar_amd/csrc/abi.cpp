// C ABI of libtpcolpar.so (declared in include/tp_colpar.h): host-side
// validation, then dispatch to the HIP kernels on the caller's stream.
// Validation runs before any HIP call, so every error path can be exercised
// on a machine without a GPU.
#include "tp_colpar.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "tp_kernels.h"

namespace {

thread_local std::string g_err;

tp_status fail(tp_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

tp_status ok()
{
    g_err.clear();
    return TP_OK;
}

tp_status hip_fail(hipError_t e, const char *what)
{
    return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The kernels address one tile's rows with 32-bit byte offsets; this bound on
// every leading dimension keeps 256 rows of bf16 (or 64 rows of fp32) under 2 GiB.
constexpr int64_t kMaxLd = int64_t(1) << 22;
constexpr int64_t kMaxM = (int64_t(1) << 31) - 1;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range span(const void *p, int64_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int element_size(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }

// Shared shape / pointer checks of the shard entry points.
tp_status check_shard(const char *fn, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_dtype dt)
{
    if (M < 0 || M > kMaxM) return fail(TP_ERR_SHAPE, "%s: M = %lld out of range [0, 2^31)", fn, (long long)M);
    if (H < 1) return fail(TP_ERR_SHAPE, "%s: H = %lld must be >= 1", fn, (long long)H);
    if (F < 1) return fail(TP_ERR_SHAPE, "%s: F = %lld must be >= 1", fn, (long long)F);
    if (T < 1 || T > TP_MAX_T) return fail(TP_ERR_SHAPE, "%s: T = %d outside [1, %d]", fn, T, TP_MAX_T);
    if (F % T != 0) return fail(TP_ERR_SHAPE, "%s: F = %lld is not divisible by T = %d", fn, (long long)F, T);
    if (i < 0 || i >= T) return fail(TP_ERR_SHAPE, "%s: shard index i = %d outside [0, %d)", fn, i, T);
    if (dt != TP_BF16 && dt != TP_F32) return fail(TP_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dt);
    return TP_OK;
}

tp_status check_dims64(const char *fn, int64_t H, int64_t F, int32_t T)
{
    const int64_t Fs = F / T;
    if (H % 64 != 0) return fail(TP_ERR_UNSUPPORTED, "%s: H = %lld is not a multiple of 64", fn, (long long)H);
    if (Fs % 64 != 0)
        return fail(TP_ERR_UNSUPPORTED, "%s: F/T = %lld is not a multiple of 64", fn, (long long)Fs);
    if (H > kMaxLd || F > kMaxLd)
        return fail(TP_ERR_UNSUPPORTED, "%s: H and F must be <= 2^22", fn);
    return TP_OK;
}

std::mutex g_cu_mu;
int g_cu[64];

int num_cu()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(g_cu_mu);
    if (g_cu[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu[dev] = n;
    }
    return g_cu[dev];
}

// ---- launches (arguments already validated) ----
tp_status run_colpar(const void *X, const void *W1t, const void *b1, void *Y_i, int64_t M, int64_t H,
                     int64_t F, int32_t T, int32_t i, tp_dtype dt, hipStream_t s)
{
    const int64_t Fs = F / T;
    const int es = element_size(dt);
    tpk::GemmArgs g;
    g.A = X;
    g.lda = H;
    g.B = static_cast<const char *>(W1t) + (int64_t)i * Fs * H * es;
    g.ldb = H;
    g.bias = b1 ? static_cast<const char *>(b1) + (int64_t)i * Fs * es : nullptr;
    g.C = Y_i;
    g.ldc = Fs;
    g.M = M;
    g.N = Fs;
    g.K = H;
    hipError_t e;
    if (dt == TP_F32)
        e = tpk::launch_gemm_f32(g, tpk::EPI_BIAS_GELU, s);
    else if (M <= 32)
        e = tpk::launch_gemv_bf16(g, tpk::EPI_BIAS_GELU, num_cu(), s);
    else
        e = tpk::launch_gemm_bf16(g, tpk::EPI_BIAS_GELU, num_cu(), s);
    return e == hipSuccess ? ok() : hip_fail(e, "tp_colpar_gelu launch");
}

tp_status run_rowpar(const void *Y_i, const void *W2t, float *Z_i, int64_t M, int64_t H, int64_t F, int32_t T,
                     int32_t i, tp_dtype dt, hipStream_t s)
{
    const int64_t Fs = F / T;
    const int es = element_size(dt);
    tpk::GemmArgs g;
    g.A = Y_i;
    g.lda = Fs;
    g.B = static_cast<const char *>(W2t) + (int64_t)i * Fs * es;
    g.ldb = F;
    g.bias = nullptr;
    g.C = Z_i;
    g.ldc = H;
    g.M = M;
    g.N = H;
    g.K = Fs;
    hipError_t e;
    if (dt == TP_F32)
        e = tpk::launch_gemm_f32(g, tpk::EPI_STORE_F32, s);
    else if (M <= 32)
        e = tpk::launch_gemv_bf16(g, tpk::EPI_STORE_F32, num_cu(), s);
    else
        e = tpk::launch_gemm_bf16(g, tpk::EPI_STORE_F32, num_cu(), s);
    return e == hipSuccess ? ok() : hip_fail(e, "tp_rowpar_partial launch");
}

tp_status validate_colpar(const char *fn, const void *X, const void *W1t, const void *b1, const void *Y_i,
                          int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_dtype dt)
{
    tp_status st = check_shard(fn, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (!X || !W1t || !Y_i) return fail(TP_ERR_NULL, "%s: X, W1t and Y_i must be non-NULL", fn);
    if ((st = check_dims64(fn, H, F, T)) != TP_OK) return st;
    if (!aligned16(X) || !aligned16(W1t) || !aligned16(Y_i) || (b1 && !aligned16(b1)))
        return fail(TP_ERR_UNSUPPORTED, "%s: X, W1t, b1 and Y_i must be 16-byte aligned", fn);
    const int es = element_size(dt);
    const Range y = span(Y_i, M * (F / T) * es);
    if (M > 0 && (overlap(y, span(X, M * H * es)) || overlap(y, span(W1t, F * H * es)) ||
                  (b1 && overlap(y, span(b1, F * es)))))
        return fail(TP_ERR_ALIAS, "%s: Y_i overlaps an input", fn);
    return TP_OK;
}

tp_status validate_rowpar(const char *fn, const void *Y_i, const void *W2t, const float *Z_i, int64_t M,
                          int64_t H, int64_t F, int32_t T, int32_t i, tp_dtype dt)
{
    tp_status st = check_shard(fn, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (!Y_i || !W2t || !Z_i) return fail(TP_ERR_NULL, "%s: Y_i, W2t and Z_i must be non-NULL", fn);
    if ((st = check_dims64(fn, H, F, T)) != TP_OK) return st;
    if (!aligned16(Y_i) || !aligned16(W2t) || !aligned16(Z_i))
        return fail(TP_ERR_UNSUPPORTED, "%s: Y_i, W2t and Z_i must be 16-byte aligned", fn);
    const int es = element_size(dt);
    const Range z = span(Z_i, M * H * 4);
    if (M > 0 && (overlap(z, span(Y_i, M * (F / T) * es)) || overlap(z, span(W2t, H * F * es))))
        return fail(TP_ERR_ALIAS, "%s: Z_i overlaps an input", fn);
    return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_colpar_gelu(const void *X, const void *W1t, const void *b1, void *Y_i, int64_t M, int64_t H,
                         int64_t F, int32_t T, int32_t i, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_colpar("tp_colpar_gelu", X, W1t, b1, Y_i, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    return run_colpar(X, W1t, b1, Y_i, M, H, F, T, i, dt, stream);
}

tp_status tp_rowpar_partial(const void *Y_i, const void *W2t, float *Z_i, int64_t M, int64_t H, int64_t F,
                            int32_t T, int32_t i, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_rowpar("tp_rowpar_partial", Y_i, W2t, Z_i, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    return run_rowpar(Y_i, W2t, Z_i, M, H, F, T, i, dt, stream);
}

tp_status tp_mlp_shard_fwd(const void *X, const void *W1t, const void *b1, const void *W2t, void *Y_ws,
                           float *Z_i, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_dtype dt,
                           hipStream_t stream)
{
    const char *fn = "tp_mlp_shard_fwd";
    tp_status st = validate_colpar(fn, X, W1t, b1, Y_ws, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if ((st = validate_rowpar(fn, Y_ws, W2t, Z_i, M, H, F, T, i, dt)) != TP_OK) return st;
    const int es = element_size(dt);
    const Range z = span(Z_i, M * H * 4), y = span(Y_ws, M * (F / T) * es);
    if (M > 0 && (overlap(z, span(X, M * H * es)) || overlap(z, span(W1t, F * H * es)) ||
                  (b1 && overlap(z, span(b1, F * es))) || overlap(y, span(W2t, H * F * es))))
        return fail(TP_ERR_ALIAS, "%s: an output overlaps an input", fn);
    if (M == 0) return ok();
    if ((st = run_colpar(X, W1t, b1, Y_ws, M, H, F, T, i, dt, stream)) != TP_OK) return st;
    return run_rowpar(Y_ws, W2t, Z_i, M, H, F, T, i, dt, stream);
}

tp_status tp_shard_reduce(const float *const *partials, int32_t T, const float *residual, float *out_f32,
                          void *out_bf16, int64_t M, int64_t H, uint32_t flags, hipStream_t stream)
{
    const char *fn = "tp_shard_reduce";
    if (T < 1 || T > TP_MAX_T) return fail(TP_ERR_SHAPE, "%s: T = %d outside [1, %d]", fn, T, TP_MAX_T);
    if (M < 0 || M > kMaxM) return fail(TP_ERR_SHAPE, "%s: M = %lld out of range", fn, (long long)M);
    if (H < 1) return fail(TP_ERR_SHAPE, "%s: H = %lld must be >= 1", fn, (long long)H);
    if (!partials || !out_f32) return fail(TP_ERR_NULL, "%s: partials and out_f32 must be non-NULL", fn);
    for (int j = 0; j < T; ++j)
        if (!partials[j]) return fail(TP_ERR_NULL, "%s: partials[%d] is NULL", fn, j);
    if (flags & ~TP_REDUCE_RMS_BF16) return fail(TP_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, flags);
    const bool rms = (flags & TP_REDUCE_RMS_BF16) != 0;
    if (rms && !out_bf16) return fail(TP_ERR_NULL, "%s: TP_REDUCE_RMS_BF16 needs out_bf16", fn);
    if (H % 4 != 0) return fail(TP_ERR_UNSUPPORTED, "%s: H = %lld is not a multiple of 4", fn, (long long)H);
    if (H > kMaxLd) return fail(TP_ERR_UNSUPPORTED, "%s: H must be <= 2^22", fn);
    bool al = aligned16(out_f32) && (!residual || aligned16(residual)) && (!out_bf16 || aligned16(out_bf16));
    for (int j = 0; j < T; ++j) al = al && aligned16(partials[j]);
    if (!al) return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    if (M > 0) {
        const Range o = span(out_f32, M * H * 4);
        const Range b = out_bf16 ? span(out_bf16, M * H * 2) : Range{0, 0};
        for (int j = 0; j < T; ++j) {
            const Range p = span(partials[j], M * H * 4);
            if (overlap(o, p) || (out_bf16 && overlap(b, p)))
                return fail(TP_ERR_ALIAS, "%s: an output overlaps partials[%d]", fn, j);
        }
        if (out_bf16 && (overlap(b, o) || (residual && overlap(b, span(residual, M * H * 4)))))
            return fail(TP_ERR_ALIAS, "%s: out_bf16 overlaps out_f32 or residual", fn);
        if (residual && residual != out_f32 && overlap(o, span(residual, M * H * 4)))
            return fail(TP_ERR_ALIAS, "%s: out_f32 partially overlaps residual", fn);
    }
    if (M == 0) return ok();
    const hipError_t e =
        tpk::launch_shard_reduce(partials, T, residual, out_f32, out_bf16, M, H, rms, TP_RMS_EPS, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "tp_shard_reduce launch");
}

const char *tp_last_error(void) { return g_err.c_str(); }

const char *tp_version(void) { return "tp_colpar 0.1.0 gfx950"; }

}  // extern "C"
