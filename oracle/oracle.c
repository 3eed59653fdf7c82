/*
 * Reference oracle for one tensor-parallel rank's share of a Megatron MLP
 * block.  TEST INFRASTRUCTURE ONLY: nothing on the product path may link,
 * load or call this file.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.
 *
 * Everything is plain fp64 C: straightforward loops, no BLAS, no blocking,
 * no fast-math, floating-point contraction off.  Inputs are the exact fp64
 * values of the (bf16- or fp32-rounded) host arrays the GPU receives.
 * Matrices are the pages' logical ones, row-major:
 *   X  [M][H]     activations
 *   W1 [H][F]     up-projection,  Y = X W1   (W1 is [in][out])
 *   b1 [F]        up-projection bias (optional)
 *   W2 [F][H]     down-projection
 * Shard i of T owns the contiguous column block C_i = [i*F/T, (i+1)*F/T)
 * of W1 and the matching row block of W2.
 *
 * Sources (page title, then section):
 *  [SLICE]  "Slice the matrix itself" (AI Engineering Visual Guide,
 *           Tensor Parallelism scene): "Column-Parallel & Row-Parallel
 *           GEMMs"; "Mathematical formulation - row-parallel matrix
 *           multiplication summation".
 *  [LESSON] "09. Tensor Parallelism in Action: Megatron-LM Matrix
 *           Splitting across NVLink & NVSwitch Networks": section 1
 *           (block split of W1 and W2, pipeline diagram), section 2,
 *           question 2 (GeLU is elementwise, so it commutes with the
 *           column split).
 *  [GUIDE]  "Tensor parallelism" (inference guide): "Concept";
 *           "Walking through a transformer block".
 *  [GELU]   Hendrycks & Gimpel, "Gaussian Error Linear Units (GELUs)",
 *           arXiv:1606.08415: the exact form x*Phi(x) and its tanh
 *           approximation.
 *  [ATTN]   Vaswani et al., "Attention Is All You Need", arXiv:1706.03762:
 *           section 3.2.1 (scaled dot-product attention), 3.2.2 (multi-head
 *           attention), 3.2.3 (the decoder masks later positions).
 *  [GQA]    Ainslie et al., "GQA: Training Generalized Multi-Query
 *           Transformer Models from Multi-Head Checkpoints",
 *           arXiv:2305.13245: groups of query heads share one key/value
 *           head.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_BAD_ARG 1

/* GeLU, tanh form [GELU]:
 *   g(x) = 0.5 * x * (1 + tanh( sqrt(2/pi) * (x + 0.044715 x^3) ))
 * The pages name GeLU without a formula ([LESSON] section 1 diagram and
 * section 2 question 2); the tanh form is the one the workloads specify. */
static double gelu_tanh(double x)
{
    const double k = sqrt(2.0 / acos(-1.0));   /* sqrt(2/pi) */
    return 0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x)));
}

/* GeLU, exact form [GELU]: g(x) = x * Phi(x) with Phi the standard normal
 * CDF, Phi(x) = (1 + erf(x / sqrt 2)) / 2; erf from the C library. */
static double gelu_erf(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

#define ORC_ACT_GELU_TANH 0
#define ORC_ACT_GELU_ERF 1
#define ORC_ACT_NONE 2

/* ORC_ACT_NONE is the identity: the column-parallel projection with no
 * activation (the attention's query, key and value projections). */
static double act_apply(int32_t act, double x)
{
    if (act == ORC_ACT_NONE) return x;
    return act == ORC_ACT_GELU_ERF ? gelu_erf(x) : gelu_tanh(x);
}

static int act_ok(int32_t act)
{
    return act == ORC_ACT_GELU_TANH || act == ORC_ACT_GELU_ERF || act == ORC_ACT_NONE;
}

void orc_gelu(int64_t n, const double *x, double *y)
{
    for (int64_t j = 0; j < n; ++j)
        y[j] = gelu_tanh(x[j]);
}

/* Either GeLU form, elementwise. */
int orc_act(int32_t act, int64_t n, const double *x, double *y)
{
    if (!act_ok(act) || n < 0 || (n > 0 && (!x || !y))) return ORC_BAD_ARG;
    for (int64_t j = 0; j < n; ++j)
        y[j] = act_apply(act, x[j]);
    return ORC_OK;
}

static int shard_ok(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i)
{
    return M >= 0 && H >= 1 && F >= 1 && T >= 1 && F % T == 0 && i >= 0 && i < T;
}

/* Column-parallel up-projection with bias and GeLU, shard i of T
 * ([SLICE] column split Y_i = X W_i; [LESSON] W1 = [W1,1 | W1,2], no
 * communication after the split; [GUIDE] "Concept": column-parallel shards
 * W along the output dimension).
 *   Y_i[m][c] = g( sum_{h=0}^{H-1} X[m][h] * W1[h][o+c]  +  b1[o+c] ),
 *   o = i*F/T,  c in [0, F/T).
 * The sum runs over h in increasing order and the bias is added last, for
 * every element, so shard outputs equal the matching columns of the
 * unsharded result bit for bit.  b1 may be NULL (no bias). */
int orc_colpar_act(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, int32_t act,
                   const double *X, const double *W1, const double *b1, double *Y_i)
{
    if (!shard_ok(M, H, F, T, i) || !act_ok(act) || !X || !W1 || !Y_i) return ORC_BAD_ARG;
    const int64_t Fs = F / T, o = (int64_t)i * Fs;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *acc = (double *)calloc((size_t)Fs, sizeof(double));
        for (int64_t h = 0; h < H; ++h) {
            const double x = X[m * H + h];
            const double *w = W1 + h * F + o;
            for (int64_t c = 0; c < Fs; ++c)
                acc[c] += x * w[c];
        }
        for (int64_t c = 0; c < Fs; ++c) {
            const double u = b1 ? acc[c] + b1[o + c] : acc[c];
            Y_i[m * Fs + c] = act_apply(act, u);
        }
        free(acc);
    }
    return ORC_OK;
}

int orc_colpar_gelu(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i,
                    const double *X, const double *W1, const double *b1,
                    double *Y_i)
{
    return orc_colpar_act(M, H, F, T, i, ORC_ACT_GELU_TANH, X, W1, b1, Y_i);
}

/* Gated first layer: the pages call the first linear layer "Gate/Up" and
 * split it by columns like W1 ([SLICE] "Column-Parallel & Row-Parallel
 * GEMMs").  Read as a gate and an up projection of the same width, both
 * split into the same column blocks, combined elementwise (so, like GeLU,
 * the combination commutes with the split):
 *   Y_i[m][c] = a( sum_h X[m][h] Wg[h][o+c] + bg[o+c] )
 *             *  ( sum_h X[m][h] Wu[h][o+c] + bu[o+c] ),   o = i*F/T,
 * with a the chosen GeLU form.  Wg, Wu are [H][F]; bg, bu may be NULL.
 * Each sum runs over h in increasing order, the bias is added last. */
int orc_colpar_gated(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, int32_t act,
                     const double *X, const double *Wg, const double *Wu,
                     const double *bg, const double *bu, double *Y_i)
{
    if (!shard_ok(M, H, F, T, i) || !act_ok(act) || act == ORC_ACT_NONE || !X || !Wg || !Wu || !Y_i)
        return ORC_BAD_ARG;
    const int64_t Fs = F / T, o = (int64_t)i * Fs;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *g = (double *)calloc((size_t)Fs, sizeof(double));
        double *u = (double *)calloc((size_t)Fs, sizeof(double));
        for (int64_t h = 0; h < H; ++h) {
            const double x = X[m * H + h];
            const double *wg = Wg + h * F + o;
            const double *wu = Wu + h * F + o;
            for (int64_t c = 0; c < Fs; ++c) {
                g[c] += x * wg[c];
                u[c] += x * wu[c];
            }
        }
        for (int64_t c = 0; c < Fs; ++c) {
            const double gate = bg ? g[c] + bg[o + c] : g[c];
            const double up = bu ? u[c] + bu[o + c] : u[c];
            Y_i[m * Fs + c] = act_apply(act, gate) * up;
        }
        free(g);
        free(u);
    }
    return ORC_OK;
}

/* Row-parallel partial product of shard i ([SLICE] "Mathematical
 * formulation - row-parallel matrix multiplication summation": Z = sum_i
 * Y_i V_i, each rank holding only its own term; [LESSON] W2 split into the
 * row blocks [W2,1 ; W2,2]; [GUIDE] row-parallel shards W along the input
 * dimension):
 *   Z_i[m][n] = sum_{c=0}^{F/T-1} Y_i[m][c] * W2[o+c][n],   o = i*F/T.
 * The same product with F := A (attention width) and Y_i := the rank's
 * slice of the attention context gives the head-sharded output projection
 * ([GUIDE] "Walking through a transformer block"). */
int orc_rowpar_partial(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i,
                       const double *Y_i, const double *W2, double *Z_i)
{
    if (!shard_ok(M, H, F, T, i) || !Y_i || !W2 || !Z_i) return ORC_BAD_ARG;
    const int64_t Fs = F / T, o = (int64_t)i * Fs;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *z = Z_i + m * H;
        for (int64_t n = 0; n < H; ++n) z[n] = 0.0;
        for (int64_t c = 0; c < Fs; ++c) {
            const double y = Y_i[m * Fs + c];
            const double *w = W2 + (o + c) * H;
            for (int64_t n = 0; n < H; ++n)
                z[n] += y * w[n];
        }
    }
    return ORC_OK;
}

/* Sum of the T row-parallel partials: what the All-Reduce-Sum delivers to
 * every rank ([SLICE] summation formula; [LESSON] one all-reduce completes
 * the MLP).  Optionally the residual stream is added ([GUIDE] both
 * all-reduces sit on residual paths):
 *   out[m][n] = (residual ? residual[m][n] : 0) + sum_{j=0}^{T-1} P_j[m][n]
 * with partials laid out [T][M][H].
 * rms_out (optional, not from the pages): the row-normalised copy
 *   rms_out[m][n] = out[m][n] / sqrt( mean_n out[m][n]^2 + eps )
 * used to keep a deep stack of blocks with no normalisation layer finite. */
int orc_shard_reduce(int32_t T, int64_t M, int64_t H, const double *partials,
                     const double *residual, double *out, double *rms_out,
                     double eps)
{
    if (T < 1 || M < 0 || H < 1 || !partials || !out) return ORC_BAD_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < H; ++n) {
            double s = 0.0;
            for (int32_t j = 0; j < T; ++j)
                s += partials[((int64_t)j * M + m) * H + n];
            out[m * H + n] = residual ? residual[m * H + n] + s : s;
        }
        if (rms_out) {
            double ss = 0.0;
            for (int64_t n = 0; n < H; ++n)
                ss += out[m * H + n] * out[m * H + n];
            const double r = 1.0 / sqrt(ss / (double)H + eps);
            for (int64_t n = 0; n < H; ++n)
                rms_out[m * H + n] = out[m * H + n] * r;
        }
    }
    return ORC_OK;
}

/* The unsharded MLP the shards reconstruct ([LESSON] pipeline diagram:
 * input, W1, GeLU, W2):  Y = g(X W1 + b1),  Z = Y W2.
 * Y [M][F] and Z [M][H] are outputs; Y may be NULL only if not wanted. */
int orc_mlp_unsharded(int64_t M, int64_t H, int64_t F,
                      const double *X, const double *W1, const double *b1,
                      const double *W2, double *Y, double *Z)
{
    if (M < 0 || H < 1 || F < 1 || !X || !W1 || !W2 || !Z) return ORC_BAD_ARG;
    double *y = Y ? Y : (double *)malloc((size_t)(M > 0 ? M : 1) * (size_t)F * sizeof(double));
    if (!y) return ORC_BAD_ARG;
    int rc = orc_colpar_gelu(M, H, F, 1, 0, X, W1, b1, y);
    if (rc == ORC_OK) rc = orc_rowpar_partial(M, H, F, 1, 0, y, W2, Z);
    if (!Y) free(y);
    return rc;
}

/* Derivative of either GeLU form ([GELU]):
 *   tanh form: g(x) = x/2 (1 + tanh v), v = c (x + a x^3), c = sqrt(2/pi),
 *              g'(x) = (1 + tanh v)/2 + x/2 (1 - tanh^2 v) c (1 + 3 a x^2);
 *   exact form: g(x) = x Phi(x), g'(x) = Phi(x) + x phi(x),
 *              phi(x) = exp(-x^2/2) / sqrt(2 pi). */
static double act_grad(int32_t act, double x)
{
    if (act == ORC_ACT_NONE) return 1.0;
    if (act == ORC_ACT_GELU_ERF) {
        const double Phi = 0.5 * (1.0 + erf(x / sqrt(2.0)));
        const double phi = exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0));
        return Phi + x * phi;
    }
    const double c = sqrt(2.0 / acos(-1.0));
    const double t = tanh(c * (x + 0.044715 * x * x * x));
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);
}

int orc_act_grad(int32_t act, int64_t n, const double *x, double *y)
{
    if (!act_ok(act) || n < 0 || (n > 0 && (!x || !y))) return ORC_BAD_ARG;
    for (int64_t k = 0; k < n; ++k) y[k] = act_grad(act, x[k]);
    return ORC_OK;
}

/* Backward pass of rank i's MLP share, given dZ [M][H], the gradient of the
 * loss at the block's output Z = sum_j Z_j.  The forward all-reduce hands
 * every rank the same dZ, and the column-parallel input's gradient needs an
 * all-reduce in the backward pass ("Slice the matrix itself", "Strict NVLink
 * Domain Constraint": all-reduces on every layer, forward and backward; the
 * "Megatron Internals II" summary on the Tensor Parallel tag page: each
 * parallel layer's contract names the gradient path that communicates).
 * With U_i = X W1[:, C_i] + b1[C_i], Y_i = g(U_i), Z_i = Y_i W2[C_i, :]:
 *   dY_i        = dZ W2[C_i, :]^T               [M][Fs]
 *   dU_i        = dY_i * g'(U_i)   (elementwise)
 *   dX_i        = dU_i W1[:, C_i]^T             [M][H]   (a partial: dX = sum_i dX_i)
 *   dW1[:, C_i] = X^T dU_i          -> dW1_i    [H][Fs]
 *   db1[C_i]    = sum_m dU_i[m][:]  -> db1_i    [Fs]
 *   dW2[C_i, :] = Y_i^T dZ          -> dW2_i    [Fs][H]
 * Every sum runs in increasing index order.  Outputs U_i, Y_i, dU_i [M][Fs]
 * may be NULL. */
int orc_mlp_shard_bwd(int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, int32_t act,
                      const double *X, const double *W1, const double *b1, const double *W2,
                      const double *dZ, double *dX_i, double *dW1_i, double *db1_i, double *dW2_i,
                      double *U_out, double *Y_out, double *dU_out)
{
    if (!shard_ok(M, H, F, T, i) || !act_ok(act) || !X || !W1 || !W2 || !dZ || !dX_i || !dW1_i ||
        !db1_i || !dW2_i)
        return ORC_BAD_ARG;
    const int64_t Fs = F / T, o = (int64_t)i * Fs;
    const size_t n = (size_t)(M > 0 ? M : 1) * (size_t)Fs;
    double *U = (double *)malloc(n * sizeof(double));
    double *Y = (double *)malloc(n * sizeof(double));
    double *dU = (double *)malloc(n * sizeof(double));
    if (!U || !Y || !dU) {
        free(U); free(Y); free(dU);
        return ORC_BAD_ARG;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t c = 0; c < Fs; ++c) {
            double u = 0.0;
            for (int64_t h = 0; h < H; ++h) u += X[m * H + h] * W1[h * F + o + c];
            if (b1) u += b1[o + c];
            U[m * Fs + c] = u;
            Y[m * Fs + c] = act_apply(act, u);
            double dy = 0.0;
            for (int64_t h = 0; h < H; ++h) dy += dZ[m * H + h] * W2[(o + c) * H + h];
            dU[m * Fs + c] = dy * act_grad(act, u);
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t h = 0; h < H; ++h) {
            double s = 0.0;
            for (int64_t c = 0; c < Fs; ++c) s += dU[m * Fs + c] * W1[h * F + o + c];
            dX_i[m * H + h] = s;
        }
    #pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h)
        for (int64_t c = 0; c < Fs; ++c) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m) s += X[m * H + h] * dU[m * Fs + c];
            dW1_i[h * Fs + c] = s;
        }
    for (int64_t c = 0; c < Fs; ++c) {
        double s = 0.0;
        for (int64_t m = 0; m < M; ++m) s += dU[m * Fs + c];
        db1_i[c] = s;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < Fs; ++c)
        for (int64_t h = 0; h < H; ++h) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m) s += Y[m * Fs + c] * dZ[m * H + h];
            dW2_i[c * H + h] = s;
        }
    if (U_out) for (size_t k = 0; k < (size_t)M * (size_t)Fs; ++k) U_out[k] = U[k];
    if (Y_out) for (size_t k = 0; k < (size_t)M * (size_t)Fs; ++k) Y_out[k] = Y[k];
    if (dU_out) for (size_t k = 0; k < (size_t)M * (size_t)Fs; ++k) dU_out[k] = dU[k];
    free(U); free(Y); free(dU);
    return ORC_OK;
}

/* Scaled dot-product attention of one rank's heads ([ATTN] 3.2.1, 3.2.2;
 * [GUIDE] "Walking through a transformer block": a rank owns a block of
 * query heads, or of GQA groups, and the matching key/value heads, so the
 * same function serves every rank on its own slices).
 *
 * Layouts, row-major: Q [Bs][Sq][nh][d], K and V [Bs][Lk][nkv][d],
 * ctx [Bs][Sq][nh][d].  Sequence b holds len_b = kv_len[b] valid keys
 * (kv_len NULL: Lk for every sequence); its Sq queries are its last Sq
 * positions, so query s sits at position p = len_b - Sq + s.  Query head h
 * reads key/value head h / G, G = nh / nkv ([GQA]: consecutive query heads
 * form a group).  Causal ([ATTN] 3.2.3, a decoder's self-attention): query
 * p sees keys t = 0..p; otherwise keys t = 0..len_b-1.
 *
 *   s_t   = ( sum_e q[e] k_t[e] ) / sqrt(d)
 *   w_t   = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
 *   ctx_e = sum_t w_t v_t[e]
 *
 * Subtracting the maximum leaves the softmax unchanged and keeps exp finite.
 * Needs 1 <= len_b <= Lk, and len_b >= Sq when causal. */
int orc_attention(int64_t Bs, int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv, int32_t d,
                  int32_t causal, const int64_t *kv_len, const double *Q, const double *K,
                  const double *V, double *ctx)
{
    if (Bs < 0 || Sq < 0 || Lk < 1 || nh < 1 || nkv < 1 || d < 1 || nh % nkv) return ORC_BAD_ARG;
    if (!Q || !K || !V || !ctx) return ORC_BAD_ARG;
    for (int64_t b = 0; b < Bs; ++b) {
        const int64_t len = kv_len ? kv_len[b] : Lk;
        if (len < 1 || len > Lk || (causal && len < Sq)) return ORC_BAD_ARG;
    }
    const int32_t G = nh / nkv;
    const double scale = 1.0 / sqrt((double)d);
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < Bs; ++b) {
        for (int64_t s = 0; s < Sq; ++s) {
            const int64_t len = kv_len ? kv_len[b] : Lk;
            const int64_t p = len - Sq + s;
            const int64_t nkeys = causal ? p + 1 : len;
            double *w = (double *)malloc((size_t)nkeys * sizeof(double));
            for (int32_t h = 0; h < nh; ++h) {
                const double *q = Q + ((b * Sq + s) * nh + h) * d;
                const int32_t g = h / G;
                double mx = -INFINITY;
                for (int64_t t = 0; t < nkeys; ++t) {
                    const double *k = K + ((b * Lk + t) * nkv + g) * d;
                    double dot = 0.0;
                    for (int32_t e = 0; e < d; ++e) dot += q[e] * k[e];
                    w[t] = dot * scale;
                    if (w[t] > mx) mx = w[t];
                }
                double den = 0.0;
                for (int64_t t = 0; t < nkeys; ++t) {
                    w[t] = exp(w[t] - mx);
                    den += w[t];
                }
                double *c = ctx + ((b * Sq + s) * nh + h) * d;
                for (int32_t e = 0; e < d; ++e) c[e] = 0.0;
                for (int64_t t = 0; t < nkeys; ++t) {
                    const double *v = V + ((b * Lk + t) * nkv + g) * d;
                    for (int32_t e = 0; e < d; ++e) c[e] += w[t] * v[e];
                }
                for (int32_t e = 0; e < d; ++e) c[e] /= den;
            }
            free(w);
        }
    }
    return ORC_OK;
}

void orc_set_threads(int32_t n) { if (n > 0) omp_set_num_threads(n); }
int32_t orc_max_threads(void) { return (int32_t)omp_get_max_threads(); }
