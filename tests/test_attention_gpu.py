"""The attention front half of one rank through the C ABI against the fp64
oracle: the column-parallel projection with no activation (tp_colpar_linear,
tp_qkv_colpar) on every kernel path, and the attention core (tp_attn_core) on
both of its kernels: the matrix-core prefill kernel (ragged query and key
counts, causal and not, grouped heads, ragged cache lengths) and the
split-key decode kernel (ragged cache lengths, grouped heads, several queries
per sequence).  Full-size shapes are checked on every decode row and on
sampled prefill rows; the whole rank chain (projection, attention, row-
parallel out-projection, reduction over ranks) against the unsharded block."""
import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colpar_amd import inputs
from tests.harness import TOL, rel_fro, to_f64, torch_dtype

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from megatron_tensor_transformer_colpar_amd import tp

D = inputs.HEAD_DIM


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def dtcode(dt):
    return tp.TP_BF16 if dt == "bf16" else tp.TP_F32


# ------------------------------------------------------ projection, no activation
@pytest.mark.parametrize("M,H,N,T,dt,pad", [
    (300, 512, 2048, 2, "bf16", 0),     # prefill GEMM, ragged M
    (130, 256, 1024, 4, "bf16", 64),    # prefill GEMM, strided output rows
    (1, 1024, 2048, 2, "bf16", 0),      # skinny-M stream
    (17, 1024, 2048, 2, "bf16", 128),   # skinny-M, two token tiles, strided output
    (8, 256, 1024, 2, "f32", 8),        # fp32 path
])
def test_colpar_linear(M, H, N, T, dt, pad):
    X, W, b, _ = inputs.mlp_inputs(inputs.Workload(60, "linear", dt, M=M, H=H, F=N, T=T), M=M)
    Ns = N // T
    ldy = Ns + pad
    for i in range(T):
        Y = torch.full((M, ldy), 7.0, dtype=torch_dtype(dt), device="cuda")
        tp.tp_colpar_linear(X.torch(), W.transposed().torch(), b.torch(), Y, ldy, M, H, N, T, i, dtcode(dt))
        torch.cuda.synchronize()
        e = rel_fro(to_f64(Y[:, :Ns]), oracle.colpar_linear(X.f64, W.f64, b.f64, T, i))
        print("  Y_%d %.2e" % (i, e))
        assert e <= TOL[dt]
        if pad:
            assert bool((Y[:, Ns:] == 7.0).all()), "wrote outside the row's N/T columns"


@pytest.mark.parametrize("M,H,nh,nkv,pad", [
    (256, 512, 8, 8, 0),     # one launch: Q, K and V as three problems of the same shape
    (8, 512, 8, 8, 0),       # skinny-M, one launch
    (96, 512, 8, 2, 0),      # grouped heads: K and V narrower, two launches
    (8, 512, 8, 4, 256),     # skinny-M, grouped, K/V rows strided as in a cache
    (8, 8192, 16, 16, 1024), # the decode shape: 3 x 64 blocks < CUs, sixteen waves per
                             # block; K/V strided as in a cache, still one launch
    (32, 8192, 16, 16, 64),  # two token tiles, sixteen waves per block
])
def test_qkv_colpar(M, H, nh, nkv, pad):
    T = 2
    A, Akv = nh * D, nkv * D
    X, Wq, Wk, Wv, bq, bk, bv = inputs.qkv_inputs(H, A, Akv, T, M=M, wid=61)
    i = 1
    As, Aks = A // T, Akv // T
    Q = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
    K = torch.empty(M, Aks + pad, dtype=torch.bfloat16, device="cuda")
    V = torch.empty(M, Aks + pad, dtype=torch.bfloat16, device="cuda")
    tp.tp_qkv_colpar(X.torch(), Wq.transposed().torch(), Wk.transposed().torch(), Wv.transposed().torch(),
                     bq.torch(), bk.torch(), bv.torch(), Q, As, K, V, Aks + pad, M, H, A, Akv, T, i)
    torch.cuda.synchronize()
    e = (rel_fro(to_f64(Q), oracle.colpar_linear(X.f64, Wq.f64, bq.f64, T, i)),
         rel_fro(to_f64(K[:, :Aks]), oracle.colpar_linear(X.f64, Wk.f64, bk.f64, T, i)),
         rel_fro(to_f64(V[:, :Aks]), oracle.colpar_linear(X.f64, Wv.f64, bv.f64, T, i)))
    print("  Q %.2e K %.2e V %.2e" % e)
    assert max(e) <= TOL["bf16"]


# ------------------------------------------------------------- attention core
def run_attn(Q, K, V, Bs, Sq, Lk, nh, nkv, causal, kv_len=None):
    """Q/K/V Synth [Bs, rows, width]; returns ctx [Bs, Sq, nh*128] as fp64."""
    dQ = Q.torch().reshape(Bs * Sq, nh * D)
    dK = K.torch().reshape(Bs * Lk, nkv * D)
    dV = V.torch().reshape(Bs * Lk, nkv * D)
    ctx = torch.full((Bs * Sq, nh * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    n = tp.tp_attn_workspace_bytes(Bs, Sq, Lk, nh, nkv)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None   # arrival counters start at zero
    lens = None if kv_len is None else torch.tensor(np.asarray(kv_len, dtype=np.int32), device="cuda")
    tp.tp_attn_core(dQ, dK, dV, ctx, lens, Bs, Sq, Lk, nh, nkv, D, nh * D, nkv * D, nh * D, causal, ws, n)
    torch.cuda.synchronize()
    return to_f64(ctx).reshape(Bs, Sq, nh * D)


@pytest.mark.parametrize("Bs,Sq,Lk,nh,nkv,causal,std", [
    (2, 200, 200, 4, 4, True, 1.0),     # ragged query tiles and key tiles
    (2, 200, 200, 4, 4, False, 1.0),
    (1, 384, 384, 2, 2, True, 2.0),     # peaked scores (std 4), three query tiles
    (2, 130, 130, 8, 2, True, 1.0),     # grouped heads, G = 4
    (3, 64, 64, 2, 1, False, 1.5),      # one key tile, G = 2
    (1, 33, 257, 2, 2, True, 1.0),      # queries are the last 33 of 257 positions
])
def test_attn_prefill(Bs, Sq, Lk, nh, nkv, causal, std):
    Q, K, V = inputs.attn_core_inputs(Bs, Sq, Lk, nh, nkv, seed=1, wid=62, q_std=std, k_std=std)
    got = run_attn(Q, K, V, Bs, Sq, Lk, nh, nkv, causal)
    want = oracle.attention(Q.f64, K.f64, V.f64, nh, nkv, causal)
    e = rel_fro(got, want)
    print("  ctx %.2e" % e)
    assert e <= TOL["bf16"]


def test_attn_prefill_ragged_cache_lengths():
    # queries are the last Sq positions of each sequence's valid keys
    Bs, Sq, Lk, nh, nkv = 3, 70, 300, 4, 2
    Q, K, V = inputs.attn_core_inputs(Bs, Sq, Lk, nh, nkv, seed=2, wid=62)
    lens = np.array([300, 70, 191], dtype=np.int32)
    for causal in (True, False):
        got = run_attn(Q, K, V, Bs, Sq, Lk, nh, nkv, causal, kv_len=lens)
        want = oracle.attention(Q.f64, K.f64, V.f64, nh, nkv, causal, kv_len=lens)
        e = rel_fro(got, want)
        print("  causal %d ctx %.2e" % (causal, e))
        assert e <= TOL["bf16"]


@pytest.mark.parametrize("Bs,Sq,Lk,nh,nkv,causal", [
    (8, 1, 2048, 8, 8, True),     # one query per sequence
    (5, 1, 700, 8, 1, True),      # grouped heads, 8 rows per key/value head
    (4, 2, 600, 8, 2, True),      # two new tokens per sequence (G * Sq = 8)
    (3, 3, 300, 2, 2, False),
    (2, 1, 64, 4, 4, False),      # a single key tile
])
def test_attn_decode(Bs, Sq, Lk, nh, nkv, causal):
    Q, K, V = inputs.attn_core_inputs(Bs, Sq, Lk, nh, nkv, seed=3, wid=63, q_std=1.5, k_std=1.5)
    lens = inputs.ragged_lengths(Bs, max(Sq, 1), Lk, seed=3)
    got = run_attn(Q, K, V, Bs, Sq, Lk, nh, nkv, causal, kv_len=lens)
    want = oracle.attention(Q.f64, K.f64, V.f64, nh, nkv, causal, kv_len=lens)
    e = rel_fro(got, want)
    print("  lens %s ctx %.2e" % (lens.tolist(), e))
    assert e <= TOL["bf16"]
    assert tp.tp_attn_workspace_bytes(Bs, Sq, Lk, nh, nkv) > 0


def test_attn_decode_workspace_reuse_counters_return_to_zero():
    # One zero-filled workspace serves decode calls of different shapes in a
    # row: the arrival counters at its end are zero again after every call,
    # and a repeated call gives the same bits (chunks merge in chunk order,
    # whichever workgroup arrives last).
    shapes = [(8, 2048, 8, 8), (1, 2048, 8, 8), (5, 700, 8, 1), (32, 512, 8, 8)]
    n_max = max(tp.tp_attn_workspace_bytes(Bs, 1, Lk, nh, nkv) for Bs, Lk, nh, nkv in shapes)
    ws = torch.zeros(n_max, dtype=torch.uint8, device="cuda")
    first = {}
    for rep in range(2):
        for Bs, Lk, nh, nkv in shapes:
            Q, K, V = inputs.attn_core_inputs(Bs, 1, Lk, nh, nkv, seed=9, wid=66, q_std=1.5, k_std=1.5)
            lens = inputs.ragged_lengths(Bs, 1, Lk, seed=9)
            ctx = torch.full((Bs, nh * D), float("nan"), dtype=torch.bfloat16, device="cuda")
            dl = torch.tensor(lens, device="cuda")
            n = tp.tp_attn_workspace_bytes(Bs, 1, Lk, nh, nkv)
            tp.tp_attn_core(Q.torch().reshape(Bs, -1), K.torch().reshape(Bs * Lk, -1), V.torch().reshape(Bs * Lk, -1),
                            ctx, dl, Bs, 1, Lk, nh, nkv, D, nh * D, nkv * D, nh * D, True, ws, n_max)
            torch.cuda.synchronize()
            assert int(ws[:16384].count_nonzero()) == 0   # the arrival counters
            got = to_f64(ctx).reshape(Bs, 1, nh * D)
            e = rel_fro(got, oracle.attention(Q.f64, K.f64, V.f64, nh, nkv, True, kv_len=lens))
            assert e <= TOL["bf16"], (Bs, Lk, nh, nkv, e)
            key = (Bs, Lk, nh, nkv)
            if rep == 0:
                first[key] = ctx.clone()
            else:
                assert torch.equal(ctx, first[key]), key
            print("  Bs=%d Lk=%d nh=%d nkv=%d: ctx %.2e" % (Bs, Lk, nh, nkv, e))


def test_attn_decode_beyond_the_counter_region_takes_the_matrix_core_kernel():
    # 520 sequences x 8 key/value heads is more (sequence, head) pairs than
    # the split-key path has arrival counters: the prefill kernel serves the
    # decode step, with no workspace
    Bs, Lk, nh = 520, 64, 8
    assert tp.tp_attn_workspace_bytes(Bs, 1, Lk, nh, nh) == 0
    Q, K, V = inputs.attn_core_inputs(Bs, 1, Lk, nh, nh, seed=12, wid=67)
    lens = inputs.ragged_lengths(Bs, 1, Lk, seed=12)
    got = run_attn(Q, K, V, Bs, 1, Lk, nh, nh, True, kv_len=lens)
    e = rel_fro(got, oracle.attention(Q.f64, K.f64, V.f64, nh, nh, True, kv_len=lens))
    print("  ctx %.2e" % e)
    assert e <= TOL["bf16"]


def test_attn_rows_without_keys_are_zero():
    # a sequence with no valid key (non-causal) and one with fewer keys than
    # causal queries: rows that see no key are written as zeros
    nh = nkv = 2
    Q, K, V = inputs.attn_core_inputs(2, 1, 128, nh, nkv, seed=4, wid=64)
    got = run_attn(Q, K, V, 2, 1, 128, nh, nkv, False, kv_len=[0, 128])
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    want = oracle.attention(Q.f64[1:], K.f64[1:], V.f64[1:], nh, nkv, False)
    assert rel_fro(got[1:], want) <= TOL["bf16"]
    Q, K, V = inputs.attn_core_inputs(1, 140, 140, nh, nkv, seed=5, wid=64)
    got = run_attn(Q, K, V, 1, 140, 140, nh, nkv, True, kv_len=[100])
    # queries 0..39 sit at negative positions; 40..139 at positions 0..99
    assert np.array_equal(got[0, :40], np.zeros_like(got[0, :40]))
    want = oracle.attention(Q.f64[:, 40:], K.f64[:, :100], V.f64[:, :100], nh, nkv, True)
    assert rel_fro(got[:, 40:], want) <= TOL["bf16"]


def test_attn_decode_rows_equal_prefill_rows():
    # the two kernels agree: decode of position p over the cache = prefill row p
    Bs, S, nh, nkv = 2, 192, 4, 4
    Q, K, V = inputs.attn_core_inputs(Bs, S, S, nh, nkv, seed=6, wid=65)
    full = run_attn(Q, K, V, Bs, S, S, nh, nkv, True)
    for p in (0, 63, 64, 191):
        Qp = inputs.Synth("bf16", np.ascontiguousarray(Q.data[:, p:p + 1]))
        one = run_attn(Qp, K, V, Bs, 1, S, nh, nkv, True, kv_len=[p + 1] * Bs)
        e = rel_fro(one[:, 0], full[:, p])
        print("  p %d: %.2e" % (p, e))
        assert e <= 2 * TOL["bf16"]


def test_attn_prefill_full_size_sampled_rows():
    # rank shard of the 8192-token prefill: 4 sequences x 2048, 8 heads
    sh = inputs.ATTN_SHAPES["prefill"]
    Q, K, V = inputs.attn_core_inputs(sh.Bs, sh.Sq, sh.Lk, sh.nh, sh.nkv, seed=7, wid=sh.wid, q_std=1.8,
                                      k_std=1.8)
    got = run_attn(Q, K, V, sh.Bs, sh.Sq, sh.Lk, sh.nh, sh.nkv, True)
    errs = []
    for b in range(sh.Bs):
        for p in inputs.row_sample(sh.Sq, 12, seed=b):
            want = oracle.attention(Q.f64[b:b + 1, p:p + 1], K.f64[b:b + 1], V.f64[b:b + 1], sh.nh, sh.nkv, True,
                                    kv_len=[p + 1])
            errs.append(rel_fro(got[b, p], want[0, 0]))
    print("  worst sampled row %.2e over %d rows" % (max(errs), len(errs)))
    assert max(errs) <= TOL["bf16"]
    assert np.isfinite(got).all()


@pytest.mark.parametrize("M", [1, 8, 32])
def test_attn_decode_full_size(M):
    # M sequences, each one new token against 2048 cached positions, 8 heads
    sh = inputs.ATTN_SHAPES["decode"]
    Q, K, V = inputs.attn_core_inputs(M, 1, sh.Lk, sh.nh, sh.nkv, seed=8, wid=sh.wid, q_std=1.8, k_std=1.8)
    got = run_attn(Q, K, V, M, 1, sh.Lk, sh.nh, sh.nkv, True)
    want = oracle.attention(Q.f64, K.f64, V.f64, sh.nh, sh.nkv, True)
    e = rel_fro(got, want)
    print("  ctx %.2e" % e)
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("Bs,S,decode", [(2, 96, False), (4, 1, True)])
def test_attention_block_shards_reduce_to_the_unsharded_block(Bs, S, decode):
    # every rank: its Q/K/V heads, attention, row-parallel out-projection;
    # the on-device sum of the partials = the unsharded attention block
    H, nh_all, T = 512, 8, 2
    A = nh_all * D
    M = Bs * S
    X, Wq, Wk, Wv, bq, bk, bv = inputs.qkv_inputs(H, A, A, T, M=M, wid=66)
    Wo = inputs.normal((A, H), 0.02, "bf16", seed=0, workload=66, tensor=inputs.WO_ID)
    dX, dWo = X.torch(), Wo.transposed().torch()
    dW = [w.transposed().torch() for w in (Wq, Wk, Wv)]
    db = [b.torch() for b in (bq, bk, bv)]
    nh = nh_all // T
    As = A // T
    parts = []
    Lk = S if not decode else 64
    caches = [(inputs.normal((Bs, Lk, As), 1.0, "bf16", seed=i, workload=66, tensor=inputs.K_ID),
               inputs.normal((Bs, Lk, As), 1.0, "bf16", seed=i, workload=66, tensor=inputs.V_ID)) for i in range(T)]
    for i in range(T):
        Qi = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
        if decode:
            # K/V caches of 64 positions; the step's token is the last one
            Ki = caches[i][0].torch().reshape(Bs * Lk, As)
            Vi = caches[i][1].torch().reshape(Bs * Lk, As)
            kv_rows_k, kv_rows_v = Ki[Lk - 1:], Vi[Lk - 1:]
            tp.tp_qkv_colpar(dX, *dW, *db, Qi, As, kv_rows_k, kv_rows_v, Lk * As, M, H, A, A, T, i)
        else:
            Ki = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
            Vi = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
            tp.tp_qkv_colpar(dX, *dW, *db, Qi, As, Ki, Vi, As, M, H, A, A, T, i)
        ctx = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
        n = tp.tp_attn_workspace_bytes(Bs, S, Lk, nh, nh)
        ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")
        tp.tp_attn_core(Qi, Ki, Vi, ctx, None, Bs, S, Lk, nh, nh, D, As, As, As, True, ws, max(n, 16))
        Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(ctx, dWo, Z, M, H, A, T, i, tp.TP_BF16)
        parts.append((Z, Ki, Vi))
    out = torch.empty(M, H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce([p[0] for p in parts], T, None, out, None, M, H)
    torch.cuda.synchronize()
    # oracle: the unsharded block over all heads, from the same cache contents
    Qf = oracle.colpar_linear(X.f64, Wq.f64, bq.f64, 1, 0).reshape(Bs, S, A)
    if decode:
        # the cached positions from their seeds, the last one from the oracle's projection
        Kf = np.concatenate([c[0].f64 for c in caches], axis=2)
        Vf = np.concatenate([c[1].f64 for c in caches], axis=2)
        Kn = oracle.colpar_linear(X.f64, Wk.f64, bk.f64, 1, 0).reshape(Bs, A)
        Vn = oracle.colpar_linear(X.f64, Wv.f64, bv.f64, 1, 0).reshape(Bs, A)
        Kg = np.concatenate([to_f64(p[1]).reshape(Bs, Lk, As) for p in parts], axis=2)
        Vg = np.concatenate([to_f64(p[2]).reshape(Bs, Lk, As) for p in parts], axis=2)
        assert np.array_equal(Kg[:, :-1], Kf[:, :-1]), "the projection wrote outside the new cache row"
        assert rel_fro(Kg[:, -1], Kn) <= TOL["bf16"] and rel_fro(Vg[:, -1], Vn) <= TOL["bf16"]
        Kf[:, -1], Vf[:, -1] = Kn, Vn
    else:
        Kf = oracle.colpar_linear(X.f64, Wk.f64, bk.f64, 1, 0).reshape(Bs, S, A)
        Vf = oracle.colpar_linear(X.f64, Wv.f64, bv.f64, 1, 0).reshape(Bs, S, A)
    ctx_all = oracle.attention(Qf, Kf, Vf, nh_all, nh_all, True).reshape(M, A)
    want = oracle.rowpar_partial(ctx_all, Wo.f64, 1, 0)
    e = rel_fro(to_f64(out), want)
    print("  block output %.2e" % e)
    assert e <= TOL["bf16"]
