// C ABI of libtpcolpar.so (declared in include/tp_colpar.h): host-side
// validation, then dispatch to the HIP kernels on the caller's stream.
// Validation runs before any HIP call, so every error path can be exercised
// on a machine without a GPU.
#include "tp_colpar.h"

#include <cstdarg>
#include <cstdint>
#include <algorithm>
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
tpk::GemmArgs empty_args()
{
    tpk::GemmArgs g{};
    g.batch = 1;
    return g;
}

hipError_t launch(const tpk::GemmArgs &g, tpk::Epilogue epi, tp_dtype dt, hipStream_t s)
{
    if (dt == TP_F32) return tpk::launch_gemm_f32(g, epi, s);
    if (g.M <= 32) return tpk::launch_gemv_bf16(g, epi, num_cu(), s);
    return tpk::launch_gemm_bf16(g, epi, num_cu(), s);
}

// Column-parallel arguments of shard i, as batch entry b.
void colpar_entry(tpk::GemmArgs &g, int b, const void *X, const void *W1t, const void *b1, void *Y_i, int64_t H,
                  int64_t Fs, int32_t i, int es)
{
    g.A[b] = X;
    g.B[b] = static_cast<const char *>(W1t) + (int64_t)i * Fs * H * es;
    g.bias[b] = b1 ? static_cast<const char *>(b1) + (int64_t)i * Fs * es : nullptr;
    g.C[b] = Y_i;
}

// Row-parallel arguments of shard i (columns C_i of W2^T), as batch entry b.
void rowpar_entry(tpk::GemmArgs &g, int b, const void *Y_i, const void *W2t, float *Z_i, int64_t Fs, int32_t i,
                  int es)
{
    g.A[b] = Y_i;
    g.B[b] = static_cast<const char *>(W2t) + (int64_t)i * Fs * es;
    g.bias[b] = nullptr;
    g.C[b] = Z_i;
}

tpk::GemmArgs colpar_args(const void *X, const void *W1t, const void *b1, void *const *Y, int nshard, int32_t i0,
                          int64_t M, int64_t H, int64_t F, int32_t T, tp_dtype dt)
{
    const int64_t Fs = F / T;
    tpk::GemmArgs g = empty_args();
    g.batch = nshard;
    for (int b = 0; b < nshard; ++b) colpar_entry(g, b, X, W1t, b1, Y[b], H, Fs, i0 + b, element_size(dt));
    g.lda = H;
    g.ldb = H;
    g.ldc = Fs;
    g.M = M;
    g.N = Fs;
    g.K = H;
    return g;
}

tp_status run_colpar(const void *X, const void *W1t, const void *b1, void *const *Y, int nshard, int32_t i0,
                     int64_t M, int64_t H, int64_t F, int32_t T, tp_dtype dt, hipStream_t s,
                     tpk::Epilogue epi = tpk::EPI_BIAS_GELU)
{
    const hipError_t e = launch(colpar_args(X, W1t, b1, Y, nshard, i0, M, H, F, T, dt), epi, dt, s);
    return e == hipSuccess ? ok() : hip_fail(e, "column-parallel launch");
}

tp_status run_rowpar(const void *const *Y, const void *W2t, float *const *Z, int nshard, int32_t i0, int64_t M,
                     int64_t H, int64_t F, int32_t T, tp_dtype dt, hipStream_t s)
{
    const int64_t Fs = F / T;
    tpk::GemmArgs g = empty_args();
    g.batch = nshard;
    for (int b = 0; b < nshard; ++b) rowpar_entry(g, b, Y[b], W2t, Z[b], Fs, i0 + b, element_size(dt));
    g.lda = Fs;
    g.ldb = F;
    g.ldc = H;
    g.M = M;
    g.N = H;
    g.K = Fs;
    const hipError_t e = launch(g, tpk::EPI_STORE_F32, dt, s);
    return e == hipSuccess ? ok() : hip_fail(e, "row-parallel launch");
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

tp_status check_act(const char *fn, tp_act act)
{
    if (act != TP_GELU_TANH && act != TP_GELU_ERF)
        return fail(TP_ERR_UNSUPPORTED, "%s: unknown activation %d", fn, (int)act);
    return TP_OK;
}

// The gated first layer: the gate operands are checked as the plain
// column-parallel call's, then the up weights and bias.
tp_status validate_gated(const char *fn, const void *X, const void *Wgt, const void *Wut, const void *bg,
                         const void *bu, const void *Y_i, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i,
                         tp_act act, tp_dtype dt)
{
    tp_status st = check_shard(fn, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (!Wut) return fail(TP_ERR_NULL, "%s: X, Wg_t, Wu_t and Y_i must be non-NULL", fn);
    if ((st = validate_colpar(fn, X, Wgt, bg, Y_i, M, H, F, T, i, dt)) != TP_OK) return st;
    if ((st = check_act(fn, act)) != TP_OK) return st;
    if (!aligned16(Wut) || (bu && !aligned16(bu)))
        return fail(TP_ERR_UNSUPPORTED, "%s: Wu_t and bu must be 16-byte aligned", fn);
    const int es = element_size(dt);
    const Range y = span(Y_i, M * (F / T) * es);
    if (M > 0 && (overlap(y, span(Wut, F * H * es)) || (bu && overlap(y, span(bu, F * es)))))
        return fail(TP_ERR_ALIAS, "%s: Y_i overlaps an input", fn);
    return TP_OK;
}

// Validation of the whole-group calls.  X/W1t (column-parallel inputs) and
// W2t (row-parallel input) may each be absent (nullptr) when the call does
// not read them; Y_ws is an output of the column-parallel step and an input
// of the row-parallel one; Z_parts may be absent.
tp_status validate_group(const char *fn, const void *X, const void *W1t, const void *b1, const void *W2t,
                         void *const *Y_ws, float *const *Z_parts, int64_t M, int64_t H, int64_t F, int32_t T,
                         tp_dtype dt)
{
    tp_status st = check_shard(fn, M, H, F, T, 0, dt);
    if (st != TP_OK) return st;
    const bool up = X || W1t, down = W2t || Z_parts;
    if ((up && (!X || !W1t)) || (down && (!W2t || !Z_parts)) || !Y_ws)
        return fail(TP_ERR_NULL, "%s: a required pointer or pointer array is NULL", fn);
    for (int j = 0; j < T; ++j)
        if (!Y_ws[j] || (Z_parts && !Z_parts[j])) return fail(TP_ERR_NULL, "%s: shard %d's buffer is NULL", fn, j);
    if ((st = check_dims64(fn, H, F, T)) != TP_OK) return st;
    bool al = (!X || aligned16(X)) && (!W1t || aligned16(W1t)) && (!W2t || aligned16(W2t)) && (!b1 || aligned16(b1));
    for (int j = 0; j < T; ++j) al = al && aligned16(Y_ws[j]) && (!Z_parts || aligned16(Z_parts[j]));
    if (!al) return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    if (M == 0) return TP_OK;
    const int es = element_size(dt);
    const int64_t Fs = F / T;
    const Range none{0, 0};
    const Range in[4] = {X ? span(X, M * H * es) : none, W1t ? span(W1t, F * H * es) : none,
                         (b1 && up) ? span(b1, F * es) : none, W2t ? span(W2t, H * F * es) : none};
    Range buf[2 * TP_MAX_T];
    int nb = 0;
    for (int j = 0; j < T; ++j) buf[nb++] = span(Y_ws[j], M * Fs * es);
    if (Z_parts)
        for (int j = 0; j < T; ++j) buf[nb++] = span(Z_parts[j], M * H * 4);
    for (int a = 0; a < nb; ++a) {
        for (const Range &r : in)
            if (overlap(buf[a], r)) return fail(TP_ERR_ALIAS, "%s: a shard buffer overlaps an input", fn);
        for (int b = a + 1; b < nb; ++b)
            if (overlap(buf[a], buf[b])) return fail(TP_ERR_ALIAS, "%s: two shard buffers overlap", fn);
    }
    return TP_OK;
}

// Column-parallel projection with no activation into Y (row stride ldy).
tp_status validate_linear(const char *fn, const void *X, const void *Wt, const void *b, const void *Y, int64_t ldy,
                          int64_t M, int64_t H, int64_t N, int32_t T, int32_t i, tp_dtype dt)
{
    tp_status st = check_shard(fn, M, H, N, T, i, dt);
    if (st != TP_OK) return st;
    if (ldy < N / T)
        return fail(TP_ERR_SHAPE, "%s: row stride %lld is below N/T = %lld", fn, (long long)ldy, (long long)(N / T));
    if (!X || !Wt || !Y) return fail(TP_ERR_NULL, "%s: X, the weight and the output must be non-NULL", fn);
    if ((st = check_dims64(fn, H, N, T)) != TP_OK) return st;
    if (ldy % 8 != 0 || ldy > kMaxLd)
        return fail(TP_ERR_UNSUPPORTED, "%s: row stride %lld must be a multiple of 8 and <= 2^22", fn, (long long)ldy);
    if (!aligned16(X) || !aligned16(Wt) || !aligned16(Y) || (b && !aligned16(b)))
        return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    if (M == 0) return TP_OK;
    const int es = element_size(dt);
    const Range y = span(Y, ((M - 1) * ldy + N / T) * es);
    if (overlap(y, span(X, M * H * es)) || overlap(y, span(Wt, N * H * es)) || (b && overlap(y, span(b, N * es))))
        return fail(TP_ERR_ALIAS, "%s: an output overlaps an input", fn);
    return TP_OK;
}

// ---- backward pass ----
// Shapes of the bf16 backward entry points: the forward's checks, plus the
// 32-bit byte offsets of the operands read along K (k-rows of up to
// max(H, F) elements, K up to max(M, H, F/T), padded by one 64-row slice).
tp_status check_bwd(const char *fn, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i)
{
    tp_status st = check_shard(fn, M, H, F, T, i, TP_BF16);
    if (st != TP_OK) return st;
    if ((st = check_dims64(fn, H, F, T)) != TP_OK) return st;
    const int64_t kmax = std::max(M, std::max(H, F / T)), ldmax = std::max(H, F);
    if ((kmax + 64) * ldmax * 2 >= (int64_t(1) << 31))
        return fail(TP_ERR_UNSUPPORTED, "%s: M, H or F too large for the kernels' 32-bit offsets", fn);
    return TP_OK;
}

// Every output range against every input range and every other output
// (nullptr entries are skipped).
tp_status check_disjoint(const char *fn, const Range *out, int nout, const Range *in, int nin)
{
    for (int a = 0; a < nout; ++a) {
        if (out[a].lo == out[a].hi) continue;
        for (int b = 0; b < nin; ++b)
            if (overlap(out[a], in[b])) return fail(TP_ERR_ALIAS, "%s: an output overlaps an input", fn);
        for (int b = a + 1; b < nout; ++b)
            if (overlap(out[a], out[b])) return fail(TP_ERR_ALIAS, "%s: two outputs overlap", fn);
    }
    return TP_OK;
}

Range span_or_none(const void *p, int64_t bytes) { return p ? span(p, bytes) : Range{0, 0}; }

hipError_t launch_mfma(tpk::GemmArgs g, tpk::Epilogue epi, tpk::Layout lay, hipStream_t s)
{
    g.layout = lay;
    return tpk::launch_gemm_bf16(g, epi, num_cu(), s);
}

constexpr int64_t kAttnMaxRowBytes = int64_t(1) << 31;   // per sequence, padded rows included

tp_status validate_attn(const char *fn, const void *Q, const void *K, const void *V, const void *ctx,
                        const int32_t *kv_len, int64_t Bs, int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv, int32_t d,
                        int64_t ldq, int64_t ldkv, int64_t ldo, int32_t causal, const void *ws, size_t ws_bytes)
{
    if (Bs < 0 || Sq < 0 || Lk < 1 || Bs > kMaxM || Sq > kMaxM || Lk > kMaxM)
        return fail(TP_ERR_SHAPE, "%s: Bs = %lld, Sq = %lld, Lk = %lld out of range", fn, (long long)Bs,
                    (long long)Sq, (long long)Lk);
    if (nh < 1 || nkv < 1 || nh > 4096 || nh % nkv != 0)
        return fail(TP_ERR_SHAPE, "%s: nh = %d, nkv = %d: need 1 <= nkv, nh <= 4096, nh %% nkv == 0", fn, nh, nkv);
    if (causal && Sq > Lk)
        return fail(TP_ERR_SHAPE, "%s: causal attention with more queries (%lld) than keys (%lld)", fn, (long long)Sq,
                    (long long)Lk);
    const int64_t A = (int64_t)nh * TP_HEAD_DIM, Akv = (int64_t)nkv * TP_HEAD_DIM;
    if (ldq < A || ldo < A || ldkv < Akv) return fail(TP_ERR_SHAPE, "%s: a row stride is below its width", fn);
    if (ldq > kMaxLd || ldo > kMaxLd || ldkv > kMaxLd) return fail(TP_ERR_SHAPE, "%s: a row stride exceeds 2^22", fn);
    if (!Q || !K || !V || !ctx) return fail(TP_ERR_NULL, "%s: Q, K, V and ctx must be non-NULL", fn);
    if (d != TP_HEAD_DIM) return fail(TP_ERR_UNSUPPORTED, "%s: head dim %d (only %d)", fn, d, TP_HEAD_DIM);
    if (ldq % 8 || ldkv % 8 || ldo % 8) return fail(TP_ERR_UNSUPPORTED, "%s: row strides must be multiples of 8", fn);
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(ctx) || (ws && !aligned16(ws)) ||
        (reinterpret_cast<uintptr_t>(kv_len) & 3u))
        return fail(TP_ERR_UNSUPPORTED, "%s: misaligned buffer", fn);
    if ((Sq + 128) * ldq * 2 >= kAttnMaxRowBytes || (Lk + 64) * ldkv * 2 >= kAttnMaxRowBytes ||
        Bs * Sq >= kMaxM || Bs * Lk >= kMaxM || Bs * nh * ((Sq + 127) / 128) >= kMaxM)
        return fail(TP_ERR_UNSUPPORTED, "%s: a sequence's rows exceed the kernels' 32-bit offsets", fn);
    const tpk::AttnPlan plan = tpk::attn_plan(Bs, Sq, Lk, nh, nkv);
    const bool need_ws = Bs > 0 && Sq > 0 && plan.decode && plan.ws_bytes > 0;
    if (need_ws && !ws) return fail(TP_ERR_NULL, "%s: this shape needs a workspace of %zu bytes", fn, plan.ws_bytes);
    if (need_ws && ws_bytes < plan.ws_bytes)
        return fail(TP_ERR_SHAPE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, plan.ws_bytes);
    if (Bs == 0 || Sq == 0) return TP_OK;
    const Range o = span(ctx, ((Bs * Sq - 1) * ldo + A) * 2);
    const Range in[4] = {span(Q, ((Bs * Sq - 1) * ldq + A) * 2), span(K, ((Bs * Lk - 1) * ldkv + Akv) * 2),
                         span(V, ((Bs * Lk - 1) * ldkv + Akv) * 2), kv_len ? span(kv_len, Bs * 4) : Range{0, 0}};
    for (const Range &r : in)
        if (overlap(o, r)) return fail(TP_ERR_ALIAS, "%s: ctx overlaps an input", fn);
    if (need_ws) {
        const Range w = span(ws, (int64_t)plan.ws_bytes);
        if (overlap(w, o)) return fail(TP_ERR_ALIAS, "%s: the workspace overlaps ctx", fn);
        for (const Range &r : in)
            if (overlap(w, r)) return fail(TP_ERR_ALIAS, "%s: the workspace overlaps an input", fn);
    }
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
    return run_colpar(X, W1t, b1, &Y_i, 1, i, M, H, F, T, dt, stream);
}

tp_status tp_colpar_act(const void *X, const void *W1t, const void *b1, void *Y_i, int64_t M, int64_t H,
                        int64_t F, int32_t T, int32_t i, tp_act act, tp_dtype dt, hipStream_t stream)
{
    const char *fn = "tp_colpar_act";
    tp_status st = validate_colpar(fn, X, W1t, b1, Y_i, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if ((st = check_act(fn, act)) != TP_OK) return st;
    if (M == 0) return ok();
    return run_colpar(X, W1t, b1, &Y_i, 1, i, M, H, F, T, dt, stream,
                      act == TP_GELU_ERF ? tpk::EPI_BIAS_GELU_ERF : tpk::EPI_BIAS_GELU);
}

tp_status tp_colpar_gated(const void *X, const void *Wgt, const void *Wut, const void *bg, const void *bu,
                          void *Y_i, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_act act,
                          tp_dtype dt, hipStream_t stream)
{
    const tp_status st =
        validate_gated("tp_colpar_gated", X, Wgt, Wut, bg, bu, Y_i, M, H, F, T, i, act, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    const int64_t Fs = F / T;
    const int es = element_size(dt);
    tpk::GemmArgs g = colpar_args(X, Wgt, bg, &Y_i, 1, i, M, H, F, T, dt);
    g.B2[0] = static_cast<const char *>(Wut) + (int64_t)i * Fs * H * es;
    g.bias2[0] = bu ? static_cast<const char *>(bu) + (int64_t)i * Fs * es : nullptr;
    const hipError_t e = launch(g, act == TP_GELU_ERF ? tpk::EPI_GATED_ERF : tpk::EPI_GATED_TANH, dt, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "gated column-parallel launch");
}

tp_status tp_rowpar_partial(const void *Y_i, const void *W2t, float *Z_i, int64_t M, int64_t H, int64_t F,
                            int32_t T, int32_t i, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_rowpar("tp_rowpar_partial", Y_i, W2t, Z_i, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    return run_rowpar(&Y_i, W2t, &Z_i, 1, i, M, H, F, T, dt, stream);
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
    if ((st = run_colpar(X, W1t, b1, &Y_ws, 1, i, M, H, F, T, dt, stream)) != TP_OK) return st;
    const void *y_in = Y_ws;
    return run_rowpar(&y_in, W2t, &Z_i, 1, i, M, H, F, T, dt, stream);
}

tp_status tp_mlp_shard_fwd_noalloc(const void *X, const void *W1t, const void *b1, const void *W2t, float *Z_i,
                                   int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_dtype dt,
                                   hipStream_t stream)
{
    static_assert(TP_NOALLOC_SCRATCH_BYTES == tpk::kScratchBytes, "header and library disagree on the limit");
    const char *fn = "tp_mlp_shard_fwd_noalloc";
    tp_status st = check_shard(fn, M, H, F, T, i, dt);
    if (st != TP_OK) return st;
    if (!X || !W1t || !W2t || !Z_i) return fail(TP_ERR_NULL, "%s: X, W1t, W2t and Z_i must be non-NULL", fn);
    if ((st = check_dims64(fn, H, F, T)) != TP_OK) return st;
    if (!aligned16(X) || !aligned16(W1t) || !aligned16(W2t) || !aligned16(Z_i) || (b1 && !aligned16(b1)))
        return fail(TP_ERR_UNSUPPORTED, "%s: X, W1t, b1, W2t and Z_i must be 16-byte aligned", fn);
    const int es = element_size(dt);
    const int64_t need = M * (F / T) * es;
    if (need > TP_NOALLOC_SCRATCH_BYTES)
        return fail(TP_ERR_UNSUPPORTED, "%s: staging Y_i needs %lld bytes, above the %lld-byte limit", fn,
                    (long long)need, (long long)TP_NOALLOC_SCRATCH_BYTES);
    const Range z = span(Z_i, M * H * 4);
    if (M > 0 && (overlap(z, span(X, M * H * es)) || overlap(z, span(W1t, F * H * es)) ||
                  (b1 && overlap(z, span(b1, F * es))) || overlap(z, span(W2t, H * F * es))))
        return fail(TP_ERR_ALIAS, "%s: Z_i overlaps an input", fn);
    if (M == 0) return ok();
    void *Y = nullptr;
    const hipError_t e = tpk::scratch_base(&Y);
    if (e != hipSuccess) return hip_fail(e, "tp_mlp_shard_fwd_noalloc: staging buffer lookup");
    if ((st = run_colpar(X, W1t, b1, &Y, 1, i, M, H, F, T, dt, stream)) != TP_OK) return st;
    const void *y_in = Y;
    return run_rowpar(&y_in, W2t, &Z_i, 1, i, M, H, F, T, dt, stream);
}

tp_status tp_colpar_gelu_group(const void *X, const void *W1t, const void *b1, void *const *Y_ws, int64_t M,
                               int64_t H, int64_t F, int32_t T, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_group("tp_colpar_gelu_group", X, W1t, b1, nullptr, Y_ws, nullptr, M, H, F, T, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    return run_colpar(X, W1t, b1, Y_ws, T, 0, M, H, F, T, dt, stream);
}

tp_status tp_rowpar_partial_group(const void *const *Y_ws, const void *W2t, float *const *Z_parts, int64_t M,
                                  int64_t H, int64_t F, int32_t T, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_group("tp_rowpar_partial_group", nullptr, nullptr, nullptr, W2t,
                                        const_cast<void *const *>(Y_ws), Z_parts, M, H, F, T, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    return run_rowpar(Y_ws, W2t, Z_parts, T, 0, M, H, F, T, dt, stream);
}

tp_status tp_mlp_group_fwd(const void *X, const void *W1t, const void *b1, const void *W2t, void *const *Y_ws,
                           float *const *Z_parts, int64_t M, int64_t H, int64_t F, int32_t T, tp_dtype dt,
                           hipStream_t stream)
{
    tp_status st = validate_group("tp_mlp_group_fwd", X, W1t, b1, W2t, Y_ws, Z_parts, M, H, F, T, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    if ((st = run_colpar(X, W1t, b1, Y_ws, T, 0, M, H, F, T, dt, stream)) != TP_OK) return st;
    return run_rowpar(reinterpret_cast<const void *const *>(Y_ws), W2t, Z_parts, T, 0, M, H, F, T, dt, stream);
}

tp_status tp_layer_fwd(float *h, void *xhat, const void *const *ctx, const void *Wot, int64_t A, const void *W1t,
                       const void *b1, const void *W2t, void *const *Y_ws, float *const *parts, int64_t M, int64_t H,
                       int64_t F, int32_t T, hipStream_t stream)
{
    const char *fn = "tp_layer_fwd";
    if (!h || !xhat || !ctx) return fail(TP_ERR_NULL, "%s: h, xhat and ctx must be non-NULL", fn);
    tp_status st = validate_group(fn, nullptr, nullptr, nullptr, Wot, const_cast<void *const *>(ctx), parts, M, H,
                                  A, T, TP_BF16);
    if (st != TP_OK) return st;
    if ((st = validate_group(fn, xhat, W1t, b1, W2t, Y_ws, parts, M, H, F, T, TP_BF16)) != TP_OK) return st;
    if (!aligned16(h) || !aligned16(xhat)) return fail(TP_ERR_UNSUPPORTED, "%s: h and xhat must be 16-byte aligned", fn);
    if (M > 0) {
        const Range rh = span(h, M * H * 4), rx = span(xhat, M * H * 2);
        const Range others[4] = {span(Wot, H * A * 2), span(W1t, F * H * 2), b1 ? span(b1, F * 2) : Range{0, 0},
                                 span(W2t, H * F * 2)};
        if (overlap(rh, rx)) return fail(TP_ERR_ALIAS, "%s: h and xhat overlap", fn);
        for (const Range &r : others)
            if (overlap(rh, r) || overlap(rx, r)) return fail(TP_ERR_ALIAS, "%s: h or xhat overlaps a weight", fn);
        for (int j = 0; j < T; ++j) {
            const Range bufs[3] = {span(ctx[j], M * (A / T) * 2), span(Y_ws[j], M * (F / T) * 2),
                                   span(parts[j], M * H * 4)};
            for (const Range &b : bufs)
                if (overlap(rh, b) || overlap(rx, b))
                    return fail(TP_ERR_ALIAS, "%s: h or xhat overlaps shard %d's buffers", fn, j);
        }
    }
    if (M == 0) return ok();
    // attention output projection of every rank, then h += sum, xhat = rms copy
    if ((st = run_rowpar(ctx, Wot, parts, T, 0, M, H, A, T, TP_BF16, stream)) != TP_OK) return st;
    hipError_t e = tpk::launch_shard_reduce(parts, T, h, h, xhat, M, H, true, TP_RMS_EPS, stream);
    if (e != hipSuccess) return hip_fail(e, "tp_layer_fwd reduce launch");
    // every rank's MLP share on xhat, then h += sum
    if ((st = run_colpar(xhat, W1t, b1, Y_ws, T, 0, M, H, F, T, TP_BF16, stream)) != TP_OK) return st;
    if ((st = run_rowpar(reinterpret_cast<const void *const *>(Y_ws), W2t, parts, T, 0, M, H, F, T, TP_BF16,
                         stream)) != TP_OK)
        return st;
    e = tpk::launch_shard_reduce(parts, T, h, h, nullptr, M, H, false, TP_RMS_EPS, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "tp_layer_fwd reduce launch");
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

tp_status tp_colpar_linear(const void *X, const void *Wt, const void *b, void *Y_i, int64_t ldy, int64_t M,
                           int64_t H, int64_t N, int32_t T, int32_t i, tp_dtype dt, hipStream_t stream)
{
    const tp_status st = validate_linear("tp_colpar_linear", X, Wt, b, Y_i, ldy, M, H, N, T, i, dt);
    if (st != TP_OK) return st;
    if (M == 0) return ok();
    tpk::GemmArgs g = colpar_args(X, Wt, b, &Y_i, 1, i, M, H, N, T, dt);
    g.ldc = ldy;
    const hipError_t e = launch(g, tpk::EPI_BIAS, dt, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "column-parallel projection launch");
}

tp_status tp_qkv_colpar(const void *X, const void *Wq_t, const void *Wk_t, const void *Wv_t, const void *bq,
                        const void *bk, const void *bv, void *Q_i, int64_t ldq, void *K_i, void *V_i, int64_t ldkv,
                        int64_t M, int64_t H, int64_t A, int64_t Akv, int32_t T, int32_t i, tp_dtype dt,
                        hipStream_t stream)
{
    const char *fn = "tp_qkv_colpar";
    tp_status st = validate_linear(fn, X, Wq_t, bq, Q_i, ldq, M, H, A, T, i, dt);
    if (st != TP_OK) return st;
    if ((st = validate_linear(fn, X, Wk_t, bk, K_i, ldkv, M, H, Akv, T, i, dt)) != TP_OK) return st;
    if ((st = validate_linear(fn, X, Wv_t, bv, V_i, ldkv, M, H, Akv, T, i, dt)) != TP_OK) return st;
    if (M == 0) return ok();
    const int es = element_size(dt);
    const Range rq = span(Q_i, ((M - 1) * ldq + A / T) * es), rk = span(K_i, ((M - 1) * ldkv + Akv / T) * es),
                rv = span(V_i, ((M - 1) * ldkv + Akv / T) * es);
    if (overlap(rq, rk) || overlap(rq, rv) || overlap(rk, rv))
        return fail(TP_ERR_ALIAS, "%s: the Q, K and V outputs overlap", fn);
    const Range wk = span(Wk_t, Akv * H * es), wv = span(Wv_t, Akv * H * es), wq = span(Wq_t, A * H * es);
    for (const Range &o : {rq, rk, rv})
        if (overlap(o, wq) || overlap(o, wk) || overlap(o, wv) || (bq && overlap(o, span(bq, A * es))) ||
            (bk && overlap(o, span(bk, Akv * es))) || (bv && overlap(o, span(bv, Akv * es))))
            return fail(TP_ERR_ALIAS, "%s: an output overlaps a weight or bias", fn);
    if (A == Akv) {
        const void *W[3] = {Wq_t, Wk_t, Wv_t}, *bias[3] = {bq, bk, bv};
        void *out[3] = {Q_i, K_i, V_i};
        tpk::GemmArgs g = colpar_args(X, Wq_t, bq, out, 1, i, M, H, A, T, dt);
        g.batch = 3;
        for (int j = 0; j < 3; ++j) colpar_entry(g, j, X, W[j], bias[j], out[j], H, A / T, i, es);
        g.ldc = ldq;
        g.ldc_b[1] = g.ldc_b[2] = ldkv;
        const hipError_t e = launch(g, tpk::EPI_BIAS, dt, stream);
        return e == hipSuccess ? ok() : hip_fail(e, "QKV projection launch");
    }
    tpk::GemmArgs gq = colpar_args(X, Wq_t, bq, &Q_i, 1, i, M, H, A, T, dt);
    gq.ldc = ldq;
    hipError_t e = launch(gq, tpk::EPI_BIAS, dt, stream);
    if (e != hipSuccess) return hip_fail(e, "query projection launch");
    void *kv[2] = {K_i, V_i};
    tpk::GemmArgs g = colpar_args(X, Wk_t, bk, kv, 1, i, M, H, Akv, T, dt);
    g.batch = 2;
    colpar_entry(g, 1, X, Wv_t, bv, V_i, H, Akv / T, i, es);
    g.ldc = ldkv;
    e = launch(g, tpk::EPI_BIAS, dt, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "key/value projection launch");
}

tp_status tp_attn_core(const void *Q, const void *K, const void *V, void *ctx, const int32_t *kv_len, int64_t Bs,
                       int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv, int32_t d, int64_t ldq, int64_t ldkv,
                       int64_t ldo, int32_t causal, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    const tp_status st = validate_attn("tp_attn_core", Q, K, V, ctx, kv_len, Bs, Sq, Lk, nh, nkv, d, ldq, ldkv, ldo,
                                       causal, workspace, ws_bytes);
    if (st != TP_OK) return st;
    if (Bs == 0 || Sq == 0) return ok();
    tpk::AttnArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = ctx;
    a.kv_len = kv_len;
    a.ldq = ldq;
    a.ldk = ldkv;
    a.ldv = ldkv;
    a.ldo = ldo;
    a.Bs = Bs;
    a.Sq = Sq;
    a.Lk = Lk;
    a.nh = nh;
    a.nkv = nkv;
    a.causal = causal != 0;
    a.ws = workspace;
    const hipError_t e = tpk::launch_attn_bf16(a, num_cu(), stream);
    return e == hipSuccess ? ok() : hip_fail(e, "attention launch");
}

size_t tp_attn_workspace_bytes(int64_t Bs, int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv)
{
    if (Bs < 1 || Sq < 1 || Lk < 1 || nh < 1 || nkv < 1 || nh % nkv != 0) return 0;
    const tpk::AttnPlan p = tpk::attn_plan(Bs, Sq, Lk, nh, nkv);
    return p.decode ? p.ws_bytes : 0;
}

tp_status tp_colpar_act_train(const void *X, const void *W1t, const void *b1, void *Y_i, void *U_i, int64_t M,
                              int64_t H, int64_t F, int32_t T, int32_t i, tp_act act, hipStream_t stream)
{
    const char *fn = "tp_colpar_act_train";
    tp_status st = validate_colpar(fn, X, W1t, b1, Y_i, M, H, F, T, i, TP_BF16);
    if (st != TP_OK) return st;
    if ((st = check_act(fn, act)) != TP_OK) return st;
    if (!U_i) return fail(TP_ERR_NULL, "%s: U_i must be non-NULL", fn);
    if (!aligned16(U_i)) return fail(TP_ERR_UNSUPPORTED, "%s: U_i must be 16-byte aligned", fn);
    const int64_t Fs = F / T;
    if (M > 0) {
        const Range u = span(U_i, M * Fs * 2);
        const Range in[4] = {span(X, M * H * 2), span(W1t, F * H * 2), span_or_none(b1, F * 2), span(Y_i, M * Fs * 2)};
        for (const Range &r : in)
            if (overlap(u, r)) return fail(TP_ERR_ALIAS, "%s: U_i overlaps another buffer", fn);
    }
    if (M == 0) return ok();
    tpk::GemmArgs g = colpar_args(X, W1t, b1, &Y_i, 1, i, M, H, F, T, TP_BF16);
    g.aux[0] = U_i;
    g.ldaux = Fs;
    // the GeLU input is kept by the MFMA GEMM's epilogue at every M
    const hipError_t e =
        launch_mfma(g, act == TP_GELU_ERF ? tpk::EPI_BIAS_GELU_ERF : tpk::EPI_BIAS_GELU, tpk::LAYOUT_KCONTIG, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "training column-parallel launch");
}

tp_status tp_rowpar_bwd(const void *dZ, const void *W2t, const void *Y_i, const void *U_i, void *dU_i, float *dW2t,
                        int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_act act, uint32_t flags,
                        hipStream_t stream)
{
    const char *fn = "tp_rowpar_bwd";
    tp_status st = check_bwd(fn, M, H, F, T, i);
    if (st != TP_OK) return st;
    if (!dZ || !W2t || !dU_i) return fail(TP_ERR_NULL, "%s: dZ, W2t and dU_i must be non-NULL", fn);
    if (dW2t && !Y_i) return fail(TP_ERR_NULL, "%s: the weight gradient needs Y_i", fn);
    if (U_i && (st = check_act(fn, act)) != TP_OK) return st;
    if (flags & ~TP_GRAD_ACCUMULATE) return fail(TP_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, flags);
    if (!aligned16(dZ) || !aligned16(W2t) || !aligned16(dU_i) || (Y_i && !aligned16(Y_i)) ||
        (U_i && !aligned16(U_i)) || (dW2t && !aligned16(dW2t)))
        return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    const int64_t Fs = F / T;
    if (M > 0) {
        const Range out[2] = {span(dU_i, M * Fs * 2), span_or_none(dW2t, H * F * 4)};
        const Range in[4] = {span(dZ, M * H * 2), span(W2t, H * F * 2), span_or_none(Y_i, M * Fs * 2),
                             span_or_none(U_i, M * Fs * 2)};
        if ((st = check_disjoint(fn, out, 2, in, 4)) != TP_OK) return st;
    }
    if (M == 0) return ok();
    // dY_i = dZ . W2[C_i,:]^T (B = columns C_i of W2^T, read along H), times g'(U_i)
    tpk::GemmArgs g = empty_args();
    g.A[0] = dZ;
    g.lda = H;
    g.B[0] = static_cast<const char *>(W2t) + (int64_t)i * Fs * 2;
    g.ldb = F;
    g.C[0] = dU_i;
    g.ldc = Fs;
    g.aux[0] = const_cast<void *>(U_i);
    g.ldaux = Fs;
    g.M = M;
    g.N = Fs;
    g.K = H;
    const tpk::Epilogue e1 = !U_i ? tpk::EPI_BIAS : act == TP_GELU_ERF ? tpk::EPI_GELU_GRAD_ERF : tpk::EPI_GELU_GRAD_TANH;
    hipError_t e = launch_mfma(g, e1, tpk::LAYOUT_B_KMAJOR, stream);
    if (e != hipSuccess) return hip_fail(e, "row-parallel input-gradient launch");
    if (!dW2t) return ok();
    // dW2[C_i,:] = Y_i^T . dZ, stored as columns C_i of dW2^T: C[h][f] = sum_m dZ[m][h] Y_i[m][f]
    tpk::GemmArgs w = empty_args();
    w.A[0] = dZ;
    w.lda = H;
    w.B[0] = Y_i;
    w.ldb = Fs;
    w.C[0] = dW2t + (int64_t)i * Fs;
    w.ldc = F;
    w.M = H;
    w.N = Fs;
    w.K = M;
    e = launch_mfma(w, (flags & TP_GRAD_ACCUMULATE) ? tpk::EPI_ACC_F32 : tpk::EPI_STORE_F32, tpk::LAYOUT_AB_KMAJOR,
                    stream);
    return e == hipSuccess ? ok() : hip_fail(e, "row-parallel weight-gradient launch");
}

tp_status tp_colpar_bwd(const void *X, const void *W1t, const void *dU_i, float *dX_i, float *dW1t, float *db1,
                        int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, uint32_t flags, hipStream_t stream)
{
    const char *fn = "tp_colpar_bwd";
    tp_status st = check_bwd(fn, M, H, F, T, i);
    if (st != TP_OK) return st;
    if (!dU_i || (dX_i && !W1t) || (dW1t && !X))
        return fail(TP_ERR_NULL, "%s: dU_i, and the inputs of each requested gradient, must be non-NULL", fn);
    if (flags & ~TP_GRAD_ACCUMULATE) return fail(TP_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, flags);
    if (!aligned16(dU_i) || (X && !aligned16(X)) || (W1t && !aligned16(W1t)) || (dX_i && !aligned16(dX_i)) ||
        (dW1t && !aligned16(dW1t)) || (db1 && !aligned16(db1)))
        return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    const int64_t Fs = F / T;
    if (M > 0) {
        const Range out[3] = {span_or_none(dX_i, M * H * 4), span_or_none(dW1t, F * H * 4), span_or_none(db1, F * 4)};
        const Range in[3] = {span_or_none(X, M * H * 2), span_or_none(W1t, F * H * 2), span(dU_i, M * Fs * 2)};
        if ((st = check_disjoint(fn, out, 3, in, 3)) != TP_OK) return st;
    }
    if (M == 0) return ok();
    const bool acc = flags & TP_GRAD_ACCUMULATE;
    hipError_t e;
    if (dX_i) {
        // dX_i = dU_i . W1[:,C_i]^T (B = rows C_i of W1^T, read along F/T): a partial over ranks
        tpk::GemmArgs g = empty_args();
        g.A[0] = dU_i;
        g.lda = Fs;
        g.B[0] = static_cast<const char *>(W1t) + (int64_t)i * Fs * H * 2;
        g.ldb = H;
        g.C[0] = dX_i;
        g.ldc = H;
        g.M = M;
        g.N = H;
        g.K = Fs;
        if ((e = launch_mfma(g, tpk::EPI_STORE_F32, tpk::LAYOUT_B_KMAJOR, stream)) != hipSuccess)
            return hip_fail(e, "column-parallel input-gradient launch");
    }
    if (dW1t) {
        // dW1[:,C_i] = X^T . dU_i, stored as rows C_i of dW1^T: C[f][h] = sum_m dU_i[m][f] X[m][h]
        tpk::GemmArgs w = empty_args();
        w.A[0] = dU_i;
        w.lda = Fs;
        w.B[0] = X;
        w.ldb = H;
        w.C[0] = dW1t + (int64_t)i * Fs * H;
        w.ldc = H;
        w.M = Fs;
        w.N = H;
        w.K = M;
        if ((e = launch_mfma(w, acc ? tpk::EPI_ACC_F32 : tpk::EPI_STORE_F32, tpk::LAYOUT_AB_KMAJOR, stream)) !=
            hipSuccess)
            return hip_fail(e, "column-parallel weight-gradient launch");
    }
    if (db1) {
        const void *x[1] = {dU_i};
        float *o[1] = {db1 + (int64_t)i * Fs};
        if ((e = tpk::launch_colsum_bf16(x, 1, Fs, M, Fs, o, acc, stream)) != hipSuccess)
            return hip_fail(e, "bias-gradient launch");
    }
    return ok();
}

tp_status tp_mlp_shard_bwd(const void *X, const void *W1t, const void *W2t, const void *U_i, const void *Y_i,
                           const void *dZ, void *dU_ws, float *dX_i, float *dW1t, float *db1, float *dW2t, int64_t M,
                           int64_t H, int64_t F, int32_t T, int32_t i, tp_act act, uint32_t flags, hipStream_t stream)
{
    const char *fn = "tp_mlp_shard_bwd";
    if (!U_i) return fail(TP_ERR_NULL, "%s: U_i must be non-NULL", fn);
    tp_status st = check_bwd(fn, M, H, F, T, i);
    if (st != TP_OK) return st;
    if (M > 0 && dU_ws) {
        const int64_t Fs = F / T;
        const Range ws = span(dU_ws, M * Fs * 2);
        const Range others[5] = {span_or_none(X, M * H * 2), span_or_none(W1t, F * H * 2), span_or_none(dX_i, M * H * 4),
                                 span_or_none(dW1t, F * H * 4), span_or_none(db1, F * 4)};
        for (const Range &r : others)
            if (overlap(ws, r)) return fail(TP_ERR_ALIAS, "%s: dU_ws overlaps another buffer", fn);
    }
    if ((st = tp_rowpar_bwd(dZ, W2t, Y_i, U_i, dU_ws, dW2t, M, H, F, T, i, act, flags, stream)) != TP_OK) {
        g_err = std::string(fn) + ": " + g_err;
        return st;
    }
    if ((st = tp_colpar_bwd(X, W1t, dU_ws, dX_i, dW1t, db1, M, H, F, T, i, flags, stream)) != TP_OK) {
        g_err = std::string(fn) + ": " + g_err;
        return st;
    }
    return ok();
}

tp_status tp_mlp_group_fwd_train(const void *X, const void *W1t, const void *b1, void *const *Y_ws, void *const *U_ws,
                                 int64_t M, int64_t H, int64_t F, int32_t T, tp_act act, hipStream_t stream)
{
    const char *fn = "tp_mlp_group_fwd_train";
    tp_status st = validate_group(fn, X, W1t, b1, nullptr, Y_ws, nullptr, M, H, F, T, TP_BF16);
    if (st != TP_OK) return st;
    if ((st = check_act(fn, act)) != TP_OK) return st;
    if (!U_ws) return fail(TP_ERR_NULL, "%s: U_ws must be non-NULL", fn);
    const int64_t Fs = F / T;
    for (int j = 0; j < T; ++j) {
        if (!U_ws[j]) return fail(TP_ERR_NULL, "%s: shard %d's U buffer is NULL", fn, j);
        if (!aligned16(U_ws[j])) return fail(TP_ERR_UNSUPPORTED, "%s: U buffers must be 16-byte aligned", fn);
    }
    if (M > 0) {
        const Range in[3] = {span(X, M * H * 2), span(W1t, F * H * 2), span_or_none(b1, F * 2)};
        for (int j = 0; j < T; ++j) {
            const Range u = span(U_ws[j], M * Fs * 2);
            for (const Range &r : in)
                if (overlap(u, r)) return fail(TP_ERR_ALIAS, "%s: a U buffer overlaps an input", fn);
            for (int k = 0; k < T; ++k)
                if (overlap(u, span(Y_ws[k], M * Fs * 2)) || (k != j && overlap(u, span(U_ws[k], M * Fs * 2))))
                    return fail(TP_ERR_ALIAS, "%s: a U buffer overlaps another shard buffer", fn);
        }
    }
    if (M == 0) return ok();
    tpk::GemmArgs g = colpar_args(X, W1t, b1, Y_ws, T, 0, M, H, F, T, TP_BF16);
    for (int j = 0; j < T; ++j) g.aux[j] = U_ws[j];
    g.ldaux = Fs;
    const hipError_t e =
        launch_mfma(g, act == TP_GELU_ERF ? tpk::EPI_BIAS_GELU_ERF : tpk::EPI_BIAS_GELU, tpk::LAYOUT_KCONTIG, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "group training column-parallel launch");
}

tp_status tp_mlp_group_bwd(const void *X, const void *W1t, const void *W2t, void *const *U_ws, void *const *Y_ws,
                           const void *dZ, void *const *dU_ws, float *const *dX_parts, float *dW1t, float *db1,
                           float *dW2t, int64_t M, int64_t H, int64_t F, int32_t T, tp_act act, uint32_t flags,
                           hipStream_t stream)
{
    const char *fn = "tp_mlp_group_bwd";
    tp_status st = check_bwd(fn, M, H, F, T, 0);
    if (st != TP_OK) return st;
    if (!X || !W1t || !W2t || !U_ws || !Y_ws || !dZ || !dU_ws || !dX_parts || !dW1t || !db1 || !dW2t)
        return fail(TP_ERR_NULL, "%s: every pointer and pointer array must be non-NULL", fn);
    for (int j = 0; j < T; ++j)
        if (!U_ws[j] || !Y_ws[j] || !dU_ws[j] || !dX_parts[j])
            return fail(TP_ERR_NULL, "%s: shard %d's buffer is NULL", fn, j);
    if ((st = check_act(fn, act)) != TP_OK) return st;
    if (flags & ~TP_GRAD_ACCUMULATE) return fail(TP_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, flags);
    bool al = aligned16(X) && aligned16(W1t) && aligned16(W2t) && aligned16(dZ) && aligned16(dW1t) &&
              aligned16(db1) && aligned16(dW2t);
    for (int j = 0; j < T; ++j)
        al = al && aligned16(U_ws[j]) && aligned16(Y_ws[j]) && aligned16(dU_ws[j]) && aligned16(dX_parts[j]);
    if (!al) return fail(TP_ERR_UNSUPPORTED, "%s: every buffer must be 16-byte aligned", fn);
    const int64_t Fs = F / T;
    if (M > 0) {
        Range out[3 + 2 * TP_MAX_T], in[4 + 2 * TP_MAX_T];
        int no = 0, ni = 0;
        out[no++] = span(dW1t, F * H * 4);
        out[no++] = span(db1, F * 4);
        out[no++] = span(dW2t, H * F * 4);
        in[ni++] = span(X, M * H * 2);
        in[ni++] = span(W1t, F * H * 2);
        in[ni++] = span(W2t, H * F * 2);
        in[ni++] = span(dZ, M * H * 2);
        for (int j = 0; j < T; ++j) {
            out[no++] = span(dU_ws[j], M * Fs * 2);
            out[no++] = span(dX_parts[j], M * H * 4);
            in[ni++] = span(U_ws[j], M * Fs * 2);
            in[ni++] = span(Y_ws[j], M * Fs * 2);
        }
        if ((st = check_disjoint(fn, out, no, in, ni)) != TP_OK) return st;
    }
    if (M == 0) return ok();
    const bool acc = flags & TP_GRAD_ACCUMULATE;
    const tpk::Epilogue wepi = acc ? tpk::EPI_ACC_F32 : tpk::EPI_STORE_F32;
    // every rank's dU_j = (dZ . W2[C_j,:]^T) * g'(U_j), one launch
    tpk::GemmArgs g = empty_args();
    g.batch = T;
    for (int j = 0; j < T; ++j) {
        g.A[j] = dZ;
        g.B[j] = static_cast<const char *>(W2t) + (int64_t)j * Fs * 2;
        g.C[j] = dU_ws[j];
        g.aux[j] = U_ws[j];
    }
    g.lda = H;
    g.ldb = F;
    g.ldc = Fs;
    g.ldaux = Fs;
    g.M = M;
    g.N = Fs;
    g.K = H;
    hipError_t e = launch_mfma(g, act == TP_GELU_ERF ? tpk::EPI_GELU_GRAD_ERF : tpk::EPI_GELU_GRAD_TANH,
                               tpk::LAYOUT_B_KMAJOR, stream);
    if (e != hipSuccess) return hip_fail(e, "group input-gradient launch");
    // dW2[C_j,:]: columns C_j of dW2^T, one launch
    tpk::GemmArgs w2 = empty_args();
    w2.batch = T;
    for (int j = 0; j < T; ++j) {
        w2.A[j] = dZ;
        w2.B[j] = Y_ws[j];
        w2.C[j] = dW2t + (int64_t)j * Fs;
    }
    w2.lda = H;
    w2.ldb = Fs;
    w2.ldc = F;
    w2.M = H;
    w2.N = Fs;
    w2.K = M;
    if ((e = launch_mfma(w2, wepi, tpk::LAYOUT_AB_KMAJOR, stream)) != hipSuccess)
        return hip_fail(e, "group weight-gradient launch");
    // dX_j = dU_j . W1[:,C_j]^T, the partials of the backward all-reduce, one launch
    tpk::GemmArgs x = empty_args();
    x.batch = T;
    for (int j = 0; j < T; ++j) {
        x.A[j] = dU_ws[j];
        x.B[j] = static_cast<const char *>(W1t) + (int64_t)j * Fs * H * 2;
        x.C[j] = dX_parts[j];
    }
    x.lda = Fs;
    x.ldb = H;
    x.ldc = H;
    x.M = M;
    x.N = H;
    x.K = Fs;
    if ((e = launch_mfma(x, tpk::EPI_STORE_F32, tpk::LAYOUT_B_KMAJOR, stream)) != hipSuccess)
        return hip_fail(e, "group input-gradient partial launch");
    // dW1[:,C_j]: rows C_j of dW1^T, one launch
    tpk::GemmArgs w1 = empty_args();
    w1.batch = T;
    for (int j = 0; j < T; ++j) {
        w1.A[j] = dU_ws[j];
        w1.B[j] = X;
        w1.C[j] = dW1t + (int64_t)j * Fs * H;
    }
    w1.lda = Fs;
    w1.ldb = H;
    w1.ldc = H;
    w1.M = Fs;
    w1.N = H;
    w1.K = M;
    if ((e = launch_mfma(w1, wepi, tpk::LAYOUT_AB_KMAJOR, stream)) != hipSuccess)
        return hip_fail(e, "group weight-gradient launch");
    // db1: the column sums of every shard's dU, one launch
    float *db1_j[tpk::kMaxPartials];
    for (int j = 0; j < T; ++j) db1_j[j] = db1 + (int64_t)j * Fs;
    if ((e = tpk::launch_colsum_bf16(dU_ws, T, Fs, M, Fs, db1_j, acc, stream)) != hipSuccess)
        return hip_fail(e, "group bias-gradient launch");
    return ok();
}

const char *tp_last_error(void) { return g_err.c_str(); }

const char *tp_version(void) { return "tp_colpar 0.1.0 gfx950"; }

}  // extern "C"
