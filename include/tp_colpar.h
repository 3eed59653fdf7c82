/*
 * tp_colpar.h -- one tensor-parallel rank's share of a Megatron MLP block on
 * MI355X (gfx950): the column-parallel up-projection with fused bias + GeLU,
 * the row-parallel down-projection (and the head-sharded attention output
 * projection) that yields an fp32 partial sum, and the on-device sum of the
 * T partials that stands in for the cross-GPU All-Reduce-Sum.
 *
 * Sources (page title, then section):
 *  [SLICE]  "Slice the matrix itself" (AI Engineering Visual Guide, Tensor
 *           Parallelism scene): "Column-Parallel & Row-Parallel GEMMs",
 *           "All-Reduce Synchronization", "Strict NVLink Domain
 *           Constraint" (all-reduces on every layer, forward and
 *           backward), "Mathematical formulation - row-parallel matrix
 *           multiplication summation".
 *  [INTERNALS] "Megatron Internals II: Column/Row Parallel Linear and Vocab
 *           Parallel Embedding" (summary on the Tensor Parallel tag page of
 *           Duo's Tech Blog): each parallel layer is a contract naming its
 *           local dimension, the collective that completes it and the
 *           gradient path that communicates.
 *  [LESSON] "09. Tensor Parallelism in Action: Megatron-LM Matrix Splitting
 *           across NVLink & NVSwitch Networks": section 1 (W1 split by
 *           columns, W2 by rows, one all-reduce, the pipeline diagram),
 *           section 2 question 2 (GeLU commutes with the column split).
 *  [GUIDE]  "Tensor parallelism" (inference guide): "Concept", "Walking
 *           through a transformer block".
 *  [GELU]   Hendrycks & Gimpel, arXiv:1606.08415 (tanh form of GeLU).
 *  [ATTN]   Vaswani et al., arXiv:1706.03762, section 3.2 (scaled
 *           dot-product and multi-head attention, the causal mask).
 *  [GQA]    Ainslie et al., arXiv:2305.13245 (grouped key/value heads).
 *
 * Notation: M tokens, hidden size H, FFN width F, TP degree T, shard index
 * i in [0, T) (the pages count ranks from 1), shard width Fs = F/T, column
 * block C_i = [i*Fs, (i+1)*Fs).  Logical weights are the pages' [in][out]
 * matrices (Y = X W).  They are STORED K-CONTIGUOUS, i.e. transposed:
 *   W1t = W1^T, row-major [F][H]   (row f holds column f of W1)
 *   W2t = W2^T, row-major [H][F]   (row h holds column h of W2)
 * All activations are row-major: X [M][H], Y_i [M][Fs], Z_i [M][H].
 *
 * Precision (tp_dtype):
 *   TP_BF16: X, W1t, b1, W2t, Y_i are bf16; products accumulate in fp32;
 *            partials Z_i and the reduction are fp32.
 *   TP_F32:  every tensor is fp32, fp32 arithmetic throughout.
 *
 * Ownership: the caller allocates, owns and frees every buffer (device
 * memory on the current HIP device, except the host array of partial
 * pointers of tp_shard_reduce).  The library allocates nothing, frees
 * nothing and never synchronizes; all work is enqueued on `stream`.
 *
 * Errors: every entry point validates its arguments on the host BEFORE any
 * HIP call and returns a tp_status; TP_ERR_HIP reports a failed launch.
 * TP_OK means "enqueued": a device fault surfaces at the caller's next
 * synchronization.  tp_last_error() gives a message for the calling thread's
 * last non-OK status.  Nothing throws or aborts across this boundary.
 *
 * Common validation (in this order):
 *   M >= 0, H >= 1, F >= 1, 1 <= T <= TP_MAX_T, F % T == 0, 0 <= i < T
 *                                                     -> TP_ERR_SHAPE
 *   required pointers non-NULL                        -> TP_ERR_NULL
 *   dtype known, H % 64 == 0, Fs % 64 == 0, every pointer 16-byte aligned
 *                                                     -> TP_ERR_UNSUPPORTED
 *   an output overlapping an input                    -> TP_ERR_ALIAS
 * M == 0 is a valid empty call: TP_OK, nothing enqueued, nothing touched.
 */
#ifndef TP_COLPAR_H
#define TP_COLPAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = 1,         /* a required pointer is NULL                  */
    TP_ERR_SHAPE = 2,        /* sizes or shard index out of range           */
    TP_ERR_UNSUPPORTED = 3,  /* valid but not supported: dtype, alignment,
                                H or F/T not a multiple of 64               */
    TP_ERR_HIP = 4,          /* a HIP call failed (message has the reason)  */
    TP_ERR_ALIAS = 5         /* an output overlaps an input                 */
} tp_status;

typedef enum { TP_BF16 = 0, TP_F32 = 1 } tp_dtype;

/* GeLU form ([GELU]): the tanh approximation (what tp_colpar_gelu applies)
 * or the exact x * Phi(x), Phi the standard normal CDF. */
typedef enum { TP_GELU_TANH = 0, TP_GELU_ERF = 1 } tp_act;

/* Largest TP degree: TP stays inside one 8-GPU node ([SLICE] "Strict
 * NVLink Domain Constraint"; [GUIDE] "Trade-off"). */
#define TP_MAX_T 8

/* tp_shard_reduce flag: also write out_bf16 = out_f32 / rms(out_f32) per row
 * (rms = sqrt(mean of squares + TP_RMS_EPS)).  Not from the pages: it keeps
 * a deep stack of blocks that has no normalisation layer finite. */
#define TP_REDUCE_RMS_BF16 1u
#define TP_RMS_EPS 1e-6f

/*
 * Column-parallel up-projection, bias and GeLU of shard i ([SLICE]
 * "Column-Parallel & Row-Parallel GEMMs"; [LESSON] section 1, no
 * communication after the column split; [LESSON] section 2 question 2: GeLU
 * is elementwise, so it is applied to the shard with no sync; [GELU]):
 *
 *   Y_i[m][c] = g( sum_h X[m][h] * W1t[i*Fs + c][h] + b1[i*Fs + c] )
 *   g(u) = u/2 * (1 + tanh( sqrt(2/pi) * (u + 0.044715 u^3) ))
 *
 *   X    [M][H]   input                                  (dtype)
 *   W1t  [F][H]   full W1^T; rows C_i are read           (dtype)
 *   b1   [F]      full bias; entries C_i are read; NULL = no bias (dtype)
 *   Y_i  [M][Fs]  output, written                        (dtype)
 * bf16: products in fp32, bias and GeLU in fp32, Y_i rounded to bf16
 * (round to nearest even).  Rank-local weights: pass the shard as the whole
 * matrix with F := Fs, T = 1, i = 0.
 */
tp_status tp_colpar_gelu(const void *X, const void *W1t, const void *b1, void *Y_i,
                         int64_t M, int64_t H, int64_t F, int32_t T, int32_t i,
                         tp_dtype dt, hipStream_t stream);

/*
 * Row-parallel partial product of shard i ([SLICE] "Column-Parallel &
 * Row-Parallel GEMMs" and the row-parallel summation: each rank's output is
 * a local partial sum; [LESSON] section 1, W2 split by rows; [GUIDE]
 * "Concept"):
 *
 *   Z_i[m][n] = sum_c Y_i[m][c] * W2t[n][i*Fs + c]
 *
 *   Y_i  [M][Fs]  input                                  (dtype)
 *   W2t  [H][F]   full W2^T; columns C_i are read (row stride F) (dtype)
 *   Z_i  [M][H]   partial, written, always fp32
 * The head-sharded attention output projection ([GUIDE] "Walking through a
 * transformer block": heads are split across ranks) is the same call with
 * Y_i := ctx_i [M][A/T] (the rank's heads, contiguous), W2t := W_o^T [H][A]
 * and F := A.
 */
tp_status tp_rowpar_partial(const void *Y_i, const void *W2t, float *Z_i,
                            int64_t M, int64_t H, int64_t F, int32_t T, int32_t i,
                            tp_dtype dt, hipStream_t stream);

/*
 * Sum of the T row-parallel partials: on one GPU this stands in for the
 * All-Reduce-Sum that completes each row-parallel projection ([SLICE]
 * summation formula and "All-Reduce Synchronization"; [LESSON] section 1:
 * one all-reduce completes the MLP; [GUIDE] the all-reduces sit on the
 * residual paths):
 *
 *   s = partials[0] + partials[1] + ... + partials[T-1]   (this order, fp32)
 *   out_f32 = residual ? residual + s : s
 *   out_bf16 (optional) = bf16(out_f32), or with TP_REDUCE_RMS_BF16
 *                         bf16(out_f32 / sqrt(mean_row(out_f32^2) + TP_RMS_EPS))
 *
 *   partials  HOST array of T device pointers, each [M][H] fp32
 *   residual  [M][H] fp32 or NULL; out_f32 may be the same buffer
 *   out_f32   [M][H] fp32, written
 *   out_bf16  [M][H] bf16 or NULL (required with TP_REDUCE_RMS_BF16)
 * Validation: 1 <= T <= TP_MAX_T, M >= 0, H >= 1 (TP_ERR_SHAPE); partials,
 * each partials[j], out_f32 non-NULL (TP_ERR_NULL); H % 4 == 0, 16-byte
 * aligned pointers, known flags (TP_ERR_UNSUPPORTED); outputs overlapping a
 * partial, or out_bf16 overlapping anything (TP_ERR_ALIAS).
 * Deterministic: fixed order, no atomics.
 */
tp_status tp_shard_reduce(const float *const *partials, int32_t T, const float *residual,
                          float *out_f32, void *out_bf16, int64_t M, int64_t H,
                          uint32_t flags, hipStream_t stream);

/*
 * A1+A2 with a choice of GeLU form ([LESSON] section 1 names GeLU, [GELU]
 * gives both forms):  Y_i = act(X . W1[:, C_i] + b1[C_i]).
 * Arguments, layouts and validation as tp_colpar_gelu, plus
 *   act not TP_GELU_TANH or TP_GELU_ERF                  -> TP_ERR_UNSUPPORTED
 * act = TP_GELU_TANH gives exactly tp_colpar_gelu's result.
 */
tp_status tp_colpar_act(const void *X, const void *W1t, const void *b1, void *Y_i, int64_t M,
                        int64_t H, int64_t F, int32_t T, int32_t i, tp_act act, tp_dtype dt,
                        hipStream_t stream);

/*
 * Gated first layer, rank i ([SLICE] "Column-Parallel & Row-Parallel GEMMs"
 * names the first linear layer "Gate/Up" and splits it by columns): a gate
 * and an up projection of width F, both split into the same column blocks,
 * combined elementwise, so no communication follows:
 *   Y_i = act(X . Wg[:, C_i] + bg[C_i]) * (X . Wu[:, C_i] + bu[C_i])
 *   Wg_t, Wu_t  Wg^T, Wu^T, each [F][H] K-contiguous like W1t
 *   bg, bu      [F] each, or NULL (no bias)
 *   Y_i         [M][Fs], input dtype; feeds tp_rowpar_partial like GeLU's Y_i
 * Validation as tp_colpar_gelu for X, Wg_t, bg, Y_i, plus Wu_t non-NULL
 * (TP_ERR_NULL), act known, Wu_t and bu 16-byte aligned (TP_ERR_UNSUPPORTED),
 * Y_i overlapping Wu_t or bu (TP_ERR_ALIAS).
 */
tp_status tp_colpar_gated(const void *X, const void *Wg_t, const void *Wu_t, const void *bg,
                          const void *bu, void *Y_i, int64_t M, int64_t H, int64_t F, int32_t T,
                          int32_t i, tp_act act, tp_dtype dt, hipStream_t stream);

/*
 * Rank i's whole MLP share ([LESSON] section 1 pipeline: input, column-
 * parallel W1, GeLU, row-parallel W2, then the all-reduce): tp_colpar_gelu
 * into the caller's workspace Y_ws [M][Fs], then tp_rowpar_partial into
 * Z_i [M][H] fp32.  Same arguments and validation as the two calls; Y_ws
 * must not overlap any other buffer.  In bf16, M <= 32 takes the
 * weight-streaming decode kernels, larger M the MFMA GEMM kernels.
 */
tp_status tp_mlp_shard_fwd(const void *X, const void *W1t, const void *b1, const void *W2t,
                           void *Y_ws, float *Z_i, int64_t M, int64_t H, int64_t F,
                           int32_t T, int32_t i, tp_dtype dt, hipStream_t stream);

/*
 * tp_mlp_shard_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same two launches, with Y_i staged in the library's own
 * device buffer instead of a caller workspace.  The caller still passes
 * every input and the output Z_i [M][H] fp32; the call allocates nothing
 * (no hipMalloc, no allocating library routine).
 *   Limit: M * F/T * (2 for TP_BF16, 4 for TP_F32) <= TP_NOALLOC_SCRATCH_BYTES
 *          (16 MiB: every decode shape; prefill up to 2048 tokens at
 *          F/T = 4096 in bf16); larger calls return TP_ERR_UNSUPPORTED
 *          before any HIP call.
 *   The buffer is one file-scope device array per GPU, held until the
 *   process ends and shared by every call on that GPU: calls on one GPU
 *   whose executions overlap (two streams, two threads) race on it and must
 *   be ordered by the caller.  Y_i is written in full before it is read, so
 *   nothing needs clearing between calls.
 * Validation as tp_mlp_shard_fwd (without Y_ws): TP_ERR_NULL for a NULL X,
 * W1t, W2t or Z_i; the shape and alignment codes of tp_colpar_gelu; Z_i
 * overlapping an input is TP_ERR_ALIAS.  The first call on a device looks up
 * the buffer's address (TP_ERR_HIP if that fails).
 */
#define TP_NOALLOC_SCRATCH_BYTES 16777216
tp_status tp_mlp_shard_fwd_noalloc(const void *X, const void *W1t, const void *b1, const void *W2t,
                                   float *Z_i, int64_t M, int64_t H, int64_t F, int32_t T,
                                   int32_t i, tp_dtype dt, hipStream_t stream);

/*
 * All T ranks' shares at once, for emulating the whole TP group on one GPU
 * ([LESSON] section 1: every rank runs the same column- then row-parallel
 * pair on its own blocks; [SLICE] summation formula: the T partials are what
 * the All-Reduce-Sum combines).  For every i in [0, T):
 *   tp_colpar_gelu_group:    Y_ws[i]    = GeLU(X . W1[:, C_i] + b1[C_i])   [M][Fs]
 *   tp_rowpar_partial_group: Z_parts[i] = Y_ws[i] . W2[C_i, :]             [M][H] fp32
 *   tp_mlp_group_fwd:        both.
 * Bit-identical to T calls of the per-shard functions, but each projection
 * is ONE launch over the tiles of all T shards, which fills the GPU when one
 * shard's tiles would not.  Y_ws and Z_parts are HOST arrays of T device
 * pointers (same dtypes and layouts as Y_i and Z_i).  Validation as the
 * per-shard calls (with i = 0), plus: every Y_ws[j] and Z_parts[j] non-NULL
 * (TP_ERR_NULL) and 16-byte aligned (TP_ERR_UNSUPPORTED); no shard buffer
 * overlapping an input or another shard buffer (TP_ERR_ALIAS).
 */
tp_status tp_colpar_gelu_group(const void *X, const void *W1t, const void *b1, void *const *Y_ws,
                               int64_t M, int64_t H, int64_t F, int32_t T, tp_dtype dt,
                               hipStream_t stream);
tp_status tp_rowpar_partial_group(const void *const *Y_ws, const void *W2t, float *const *Z_parts,
                                  int64_t M, int64_t H, int64_t F, int32_t T, tp_dtype dt,
                                  hipStream_t stream);
tp_status tp_mlp_group_fwd(const void *X, const void *W1t, const void *b1, const void *W2t,
                           void *const *Y_ws, float *const *Z_parts, int64_t M, int64_t H, int64_t F,
                           int32_t T, tp_dtype dt, hipStream_t stream);

/*
 * One block of a layer stack, with the whole TP group emulated on one GPU
 * (bf16 storage, fp32 residual stream).  The two all-reduces of a layer
 * follow the attention output projection and the MLP and sit on the
 * residual paths ([SLICE] "All-Reduce Synchronization"; [GUIDE] "Walking
 * through a transformer block"):
 *   parts[i] = ctx[i] . W_o[A_i, :]                 (head-sharded out-proj)
 *   h       += parts[0] + ... + parts[T-1]
 *   xhat     = bf16(h / sqrt(mean_row(h^2) + TP_RMS_EPS))   (not from the
 *              pages: keeps a deep stack with no normalisation layer finite)
 *   Y_ws[i]  = GeLU(xhat . W1[:, C_i] + b1[C_i]),  parts[i] = Y_ws[i] . W2[C_i, :]
 *   h       += parts[0] + ... + parts[T-1]
 *   h      [M][H] fp32, read and written (the residual stream)
 *   xhat   [M][H] bf16 workspace (written)
 *   ctx    HOST array of T device pointers, each [M][A/T] bf16 (rank i's heads)
 *   Wot    W_o^T [H][A] bf16;  W1t, b1, W2t as tp_mlp_group_fwd
 *   Y_ws, parts  HOST arrays of T workspaces ([M][F/T] bf16, [M][H] fp32)
 * Validation: as tp_mlp_group_fwd for the MLP and for the out-projection
 * (with F := A), plus h, xhat non-NULL and 16-byte aligned and disjoint from
 * every other buffer.
 */
tp_status tp_layer_fwd(float *h, void *xhat, const void *const *ctx, const void *Wot, int64_t A,
                       const void *W1t, const void *b1, const void *W2t, void *const *Y_ws,
                       float *const *parts, int64_t M, int64_t H, int64_t F, int32_t T,
                       hipStream_t stream);

/*
 * ---- The attention front half of rank i ----
 * [GUIDE] "Walking through a transformer block": attention is sharded by
 * heads (or by GQA groups of heads) across the TP ranks, and the KV cache
 * is sharded along heads, so rank i projects and attends over its own heads
 * only and its context ctx_i feeds the row-parallel out-projection
 * (tp_rowpar_partial with F := A).  The attention itself is the published
 * scaled dot-product attention ([ATTN] Vaswani et al., arXiv:1706.03762,
 * sections 3.2.1-3.2.3, the decoder's causal mask) with grouped key/value
 * heads ([GQA] Ainslie et al., arXiv:2305.13245).  Head dim TP_HEAD_DIM.
 */
#define TP_HEAD_DIM 128

/*
 * Column-parallel projection with no activation ([SLICE] column split;
 * rank i's block C_i of the N output columns):
 *   Y_i[m][c] = sum_h X[m][h] * W[h][i*N/T + c] + b[i*N/T + c]
 *   Wt   W^T, [N][H] K-contiguous (full matrix); b [N] or NULL
 *   Y_i  M rows of N/T in the input dtype, row stride ldy >= N/T elements
 *        (lets the key and value rows of a decode step land in a cache)
 * Validation as tp_colpar_gelu with F := N, plus ldy >= N/T and ldy % 8 == 0
 * (TP_ERR_SHAPE / TP_ERR_UNSUPPORTED).
 */
tp_status tp_colpar_linear(const void *X, const void *Wt, const void *b, void *Y_i, int64_t ldy,
                           int64_t M, int64_t H, int64_t N, int32_t T, int32_t i, tp_dtype dt,
                           hipStream_t stream);

/*
 * Rank i's query, key and value projections in one call:
 *   Q_i = X Wq[:, Aq_i] + bq[Aq_i]   [M][A/T],   row stride ldq
 *   K_i = X Wk[:, Ak_i] + bk[Ak_i]   [M][Akv/T], row stride ldkv
 *   V_i = X Wv[:, Ak_i] + bv[Ak_i]   [M][Akv/T], row stride ldkv
 * A = nh * TP_HEAD_DIM (query width), Akv = nkv * TP_HEAD_DIM (key/value
 * width; Akv == A without grouping); Wq_t [A][H], Wk_t and Wv_t [Akv][H]
 * K-contiguous; biases [A] / [Akv] or NULL.  One launch when A == Akv,
 * else two.  Validation as tp_colpar_linear for each of the
 * three, plus the three outputs pairwise disjoint (TP_ERR_ALIAS).
 */
tp_status tp_qkv_colpar(const void *X, const void *Wq_t, const void *Wk_t, const void *Wv_t,
                        const void *bq, const void *bk, const void *bv, void *Q_i, int64_t ldq,
                        void *K_i, void *V_i, int64_t ldkv, int64_t M, int64_t H, int64_t A,
                        int64_t Akv, int32_t T, int32_t i, tp_dtype dt, hipStream_t stream);

/*
 * Scaled dot-product attention of one rank's heads, bf16 in and out, fp32
 * scores, softmax and accumulation ([ATTN] 3.2.1-3.2.3, [GQA]):
 *   ctx = softmax(q k^T / sqrt(d) over the visible keys) v   per query head
 *   Q    [Bs*Sq][ldq]:  row b*Sq + s = query s of sequence b; query head h
 *        at columns h*TP_HEAD_DIM (nh heads)
 *   K, V [Bs*Lk][ldkv]: row b*Lk + t = key/value t of sequence b (its
 *        cache of capacity Lk); head g at columns g*TP_HEAD_DIM (nkv heads)
 *   ctx  [Bs*Sq][ldo], laid out like Q
 *   kv_len  device int32 [Bs], the valid keys of each sequence, or NULL
 *        (every sequence holds Lk); read on the device, values clamped to
 *        [0, Lk]
 * The Sq queries of sequence b are its last Sq positions: query s sits at
 * position kv_len[b] - Sq + s.  causal != 0: it sees keys 0 .. its position;
 * causal == 0: keys 0 .. kv_len[b]-1.  Query head h reads key/value head
 * h / (nh / nkv).  A query row that sees no key is written as zeros.
 * When G*Sq <= 8 (G = nh/nkv) and Bs*nkv <= 4096 the keys are split over
 * many workgroups of one launch, and the last workgroup of each (sequence,
 * key/value head) to finish merges the chunks (in chunk order: the result
 * does not depend on which one finishes last).  That path needs
 * `workspace`, a device buffer of at least
 * tp_attn_workspace_bytes(Bs, Sq, Lk, nh, nkv) bytes: 4096 arrival counters
 * (16 KiB) at its start, then the chunks' partials.  The counters must be
 * zero when the workspace is first used (allocate it zero-filled); every
 * call returns them to zero, so the buffer can serve any later call, of any
 * shape, whose work is ordered after this one's (calls that overlap in time
 * must not share a workspace).  Otherwise the workspace is not touched and
 * may be NULL.
 * Validation: Bs, Sq >= 0, Lk >= 1, nh, nkv >= 1, nh % nkv == 0, causal
 * needs Sq <= Lk, ldq and ldo >= nh*128, ldkv >= nkv*128 (TP_ERR_SHAPE);
 * Q, K, V, ctx non-NULL, workspace non-NULL when needed (TP_ERR_NULL);
 * d == TP_HEAD_DIM, strides multiples of 8, Q, K, V, ctx and workspace
 * 16-byte aligned, kv_len 4-byte aligned, Sq*ldq and Lk*ldkv below 2^30
 * (TP_ERR_UNSUPPORTED); ws_bytes too small (TP_ERR_SHAPE); ctx or workspace
 * overlapping an input or each other (TP_ERR_ALIAS).  Bs == 0 or Sq == 0 is
 * an empty call.
 */
tp_status tp_attn_core(const void *Q, const void *K, const void *V, void *ctx, const int32_t *kv_len,
                       int64_t Bs, int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv, int32_t d,
                       int64_t ldq, int64_t ldkv, int64_t ldo, int32_t causal, void *workspace,
                       size_t ws_bytes, hipStream_t stream);

/* Workspace bytes tp_attn_core needs for these sizes (0: none), counters
 * included.  Depends on the sizes only, not on the device. */
size_t tp_attn_workspace_bytes(int64_t Bs, int64_t Sq, int64_t Lk, int32_t nh, int32_t nkv);

/*
 * ---- Backward pass of rank i's share (bf16; gradients in fp32) ----
 * [SLICE] "Strict NVLink Domain Constraint": all-reduces run on every
 * layer in the forward and the backward pass; [INTERNALS]: each layer's
 * contract names the gradient path that communicates.  The forward's
 * All-Reduce-Sum gives every rank the same output gradient dZ, and the
 * column-parallel layer's input gradient is a partial sum that the backward
 * all-reduce completes (on one GPU: tp_shard_reduce over the ranks' dX_i);
 * the weight and bias gradients of a rank are its own blocks, with no
 * communication.  With U_i = X W1[:,C_i] + b1[C_i] (the GeLU input) and
 * Y_i = g(U_i):
 *   dU_i        = (dZ W2[C_i,:]^T) * g'(U_i)
 *   dX_i        = dU_i W1[:,C_i]^T            (partial; dX = sum_i dX_i)
 *   dW1[:,C_i]  = X^T dU_i,   db1[C_i] = sum over tokens of dU_i
 *   dW2[C_i,:]  = Y_i^T dZ
 * Gradients are stored like the weights (dW1t = dW1^T [F][H], dW2t = dW2^T
 * [H][F], db1 [F], all fp32); rank i writes only its blocks.  With
 * TP_GRAD_ACCUMULATE they are added to the buffers' contents instead
 * (gradient accumulation over micro-batches).  M == 0 enqueues nothing and
 * writes nothing.  Validation: the forward's shape checks (F % T, H and F/T
 * multiples of 64, ...) plus (max(M, H, F/T) + 64) * max(H, F) < 2^30
 * (TP_ERR_UNSUPPORTED), unknown flags (TP_ERR_UNSUPPORTED), outputs
 * overlapping inputs or each other (TP_ERR_ALIAS).
 */
#define TP_GRAD_ACCUMULATE 1u

/*
 * Training forward of the column-parallel up-projection: tp_colpar_act in
 * bf16, and the GeLU input U_i [M][F/T] (bf16) is kept for the backward.
 */
tp_status tp_colpar_act_train(const void *X, const void *W1t, const void *b1, void *Y_i, void *U_i,
                              int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_act act,
                              hipStream_t stream);

/*
 * Backward of rank i's row-parallel projection (A3; the head-sharded
 * out-projection A4 with F := A and U_i = NULL):
 *   dU_i [M][F/T] bf16 = (dZ . W2[C_i,:]^T) * g'(U_i), or without U_i the
 *                        plain input gradient dZ . W2[C_i,:]^T
 *   dW2t columns C_i   = (Y_i^T . dZ)^T  (fp32, written or accumulated);
 *                        dW2t may be NULL (then Y_i may be NULL too)
 *   dZ [M][H] bf16, W2t [H][F] bf16, Y_i and U_i [M][F/T] bf16.
 */
tp_status tp_rowpar_bwd(const void *dZ, const void *W2t, const void *Y_i, const void *U_i, void *dU_i,
                        float *dW2t, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_act act,
                        uint32_t flags, hipStream_t stream);

/*
 * Backward of rank i's column-parallel projection (A1+A2), from the
 * gradient at its output dU_i [M][F/T] bf16 (the GeLU input's, from
 * tp_rowpar_bwd):
 *   dX_i [M][H] fp32 = dU_i . W1[:,C_i]^T          (may be NULL)
 *   dW1t rows C_i    = (X^T . dU_i)^T, fp32 [F][H]  (may be NULL)
 *   db1[C_i]         = column sums of dU_i, fp32 [F] (may be NULL)
 */
tp_status tp_colpar_bwd(const void *X, const void *W1t, const void *dU_i, float *dX_i, float *dW1t,
                        float *db1, int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, uint32_t flags,
                        hipStream_t stream);

/*
 * Rank i's whole backward: tp_rowpar_bwd into the caller's workspace dU_ws
 * [M][F/T] bf16, then tp_colpar_bwd from it.  U_i and Y_i come from
 * tp_colpar_act_train.
 */
tp_status tp_mlp_shard_bwd(const void *X, const void *W1t, const void *W2t, const void *U_i, const void *Y_i,
                           const void *dZ, void *dU_ws, float *dX_i, float *dW1t, float *db1, float *dW2t,
                           int64_t M, int64_t H, int64_t F, int32_t T, int32_t i, tp_act act, uint32_t flags,
                           hipStream_t stream);

/*
 * The whole TP group's training forward and backward on one GPU (the
 * emulation of every rank, as tp_mlp_group_fwd; [LESSON] section 1), one
 * launch per projection over the tiles of all T ranks:
 *   tp_mlp_group_fwd_train: Y_ws[j] = g(U_ws[j]), U_ws[j] = X W1[:,C_j] + b1[C_j]
 *   tp_mlp_group_bwd: for every rank j, dU_ws[j] = (dZ W2[C_j,:]^T) * g'(U_ws[j]),
 *     dX_parts[j] = dU_ws[j] W1[:,C_j]^T (fp32 partials: tp_shard_reduce of
 *     them is the backward all-reduce), and the whole dW1t [F][H], db1 [F],
 *     dW2t [H][F] (fp32, written or accumulated: every rank's block).
 * U_ws, Y_ws, dU_ws, dX_parts: HOST arrays of T device pointers.
 * Validation: as tp_mlp_group_fwd and the per-rank backward entry points;
 * every pointer non-NULL (TP_ERR_NULL); no output overlapping an input or
 * another output (TP_ERR_ALIAS).
 */
tp_status tp_mlp_group_fwd_train(const void *X, const void *W1t, const void *b1, void *const *Y_ws,
                                 void *const *U_ws, int64_t M, int64_t H, int64_t F, int32_t T, tp_act act,
                                 hipStream_t stream);
tp_status tp_mlp_group_bwd(const void *X, const void *W1t, const void *W2t, void *const *U_ws,
                           void *const *Y_ws, const void *dZ, void *const *dU_ws, float *const *dX_parts,
                           float *dW1t, float *db1, float *dW2t, int64_t M, int64_t H, int64_t F, int32_t T,
                           tp_act act, uint32_t flags, hipStream_t stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *tp_last_error(void);

/* Library version string. */
const char *tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_COLPAR_H */
