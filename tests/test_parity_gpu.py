"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case runs the library on seeded inputs and the oracle on the same host
arrays; the bar is a relative Frobenius error of 5e-3 for bf16 storage with
fp32 accumulation and 1e-5 for fp32 (per checked tensor: each Y_i, Z_i and
the reduced Z).  Full-size workloads are checked on a seeded sample of token
rows (no step of the block mixes rows, so a row's outputs depend only on that
row's inputs).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colpar_amd import inputs
from tests.harness import TOL, DeviceMLP, rel_fro, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from megatron_tensor_transformer_colpar_amd import tp


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def check_all_shards(w, M, T, rows=None, seed=0, use_fused=True, shard_ids=None):
    """Run every shard of workload w and the reduce; compare (sampled) rows."""
    X, W1, b1, W2 = inputs.mlp_inputs(w, M=M, seed=seed)
    dev = DeviceMLP(X, W1, b1, W2)
    parts, Z = dev.all_shards_reduced(T, use_fused)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    Xr = X.f64[rows]
    tol = TOL[w.dtype]
    zs = []
    for i in range(T):
        Yr, Zr = oracle.mlp_shard(Xr, W1.f64, b1.f64, W2.f64, T, i)
        zs.append(Zr)
        ey = rel_fro(to_f64(parts[i][0])[rows], Yr)
        ez = rel_fro(to_f64(parts[i][1])[rows], Zr)
        print("  shard %d: Y_i %.2e  Z_i %.2e" % (i, ey, ez))
        assert ey <= tol and ez <= tol, (i, ey, ez)
    ez = rel_fro(to_f64(Z)[rows], oracle.shard_reduce(np.stack(zs)))
    _, Zu = oracle.mlp_unsharded(Xr, W1.f64, b1.f64, W2.f64)
    eu = rel_fro(to_f64(Z)[rows], Zu)
    print("  reduced Z: vs sum of oracle partials %.2e, vs unsharded %.2e" % (ez, eu))
    assert ez <= tol and eu <= tol
    return parts, Z


# ------------------------------------------------------------- fp32 mode
def test_tiny_f32_two_ranks():
    # X[8,256], W1[256,1024] split in 2, b1 = 0, W2[1024,256] split in 2.
    check_all_shards(inputs.WORKLOADS["tiny_f32"], M=8, T=2)


def test_tiny_f32_with_bias_and_separate_calls():
    w = inputs.Workload(1, "tiny_f32_bias", "f32", M=8, H=256, F=1024, T=2, b_std=0.01)
    check_all_shards(w, M=8, T=2, use_fused=False)


def test_f32_ragged_multi_tile():
    w = inputs.Workload(11, "f32_ragged", "f32", M=70, H=192, F=512, T=4)
    check_all_shards(w, M=70, T=4)


# ------------------------------------------------------- bf16 GEMM path
def test_bf16_ragged_all_shards():
    # M = 300 (ragged in M), shard width 320 (ragged against 128/256 tiles)
    w = inputs.Workload(12, "bf16_ragged", "bf16", M=300, H=512, F=1280, T=4)
    check_all_shards(w, M=300, T=4)


def test_bf16_smallest_gemm_m():
    # M = 33 is the first size that takes the MFMA GEMM rather than the decode path
    w = inputs.Workload(13, "bf16_m33", "bf16", M=33, H=256, F=512, T=2)
    check_all_shards(w, M=33, T=2, use_fused=False)


def tile_row_sample(M, extra, seed=0):
    """First and last row of every 256-row tile row, plus `extra` seeded rows:
    a wrong tile row anywhere shows in the sample."""
    ends = {r for t in range(0, M, 256) for r in (t, min(M, t + 256) - 1)}
    return np.array(sorted(ends | set(inputs.row_sample(M, extra, seed=seed).tolist())), dtype=np.int64)


def per_block(got, want, rows, what):
    """rel-Frobenius of each 256-row block of the sample (each <= the bf16 bar)."""
    worst = 0.0
    for b in np.unique(rows // 256):
        sel = rows // 256 == b
        e = rel_fro(got[sel], want[sel])
        assert e <= TOL["bf16"], (what, int(b), e)
        worst = max(worst, e)
    return worst


def test_gpt_block_shard_full_size_sampled_rows():
    # H=4096, F=16384, T=4, M=2048: all 4 shards and the reduce, as benchmarked;
    # both ends of every 256-row tile row plus 16 seeded rows
    w = inputs.WORKLOADS["gpt_block_shard"]
    check_all_shards(w, M=w.M, T=w.T, rows=tile_row_sample(w.M, 16))


def test_prefill_full_size_every_tile_row():
    # H=8192, F=32768, T=8: rank 0's own weight blocks (F := F/T, T := 1),
    # M=8192, the launch configuration the bench times: the first and last row
    # of each of the 32 tile rows plus 64 seeded rows, error per 256-row block
    w = inputs.WORKLOADS["prefill"]
    X, W1, b1, W2 = inputs.mlp_inputs(w, shard_only=0)
    dev = DeviceMLP(X, W1, b1, W2)
    Y, Z = dev.shard(1, 0, use_fused=False)
    torch.cuda.synchronize()
    rows = tile_row_sample(w.M, 64)
    Yr, Zr = oracle.mlp_shard(X.f64[rows], W1.f64, b1.f64, W2.f64, 1, 0)
    Yg, Zg = to_f64(Y)[rows], to_f64(Z)[rows]
    ey, ez = rel_fro(Yg, Yr), rel_fro(Zg, Zr)
    by, bz = per_block(Yg, Yr, rows, "Y"), per_block(Zg, Zr, rows, "Z")
    print("  %d rows: Y_0 %.2e  Z_0 %.2e  (worst 256-row block: Y %.2e  Z %.2e)" % (len(rows), ey, ez, by, bz))
    assert ey <= TOL["bf16"] and ez <= TOL["bf16"]
    # the fused entry point computes the same bits
    Y2, Z2 = dev.shard(1, 0, use_fused=True)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2) and torch.equal(Z, Z2)


@pytest.mark.parametrize("M,H,Fs", [(4196, 4096, 4096), (4096, 4160, 4160)])
@pytest.mark.parametrize("train", [False, True])
def test_ragged_tokens_on_the_largest_tile(train, M, H, Fs):
    # 272 tiles either way, so both projections run the 256x256 tile, whose
    # epilogues stage through LDS: 4196 tokens (16 whole 256-row tiles and
    # 100 rows) store a partial last tile row; H = F/T = 4160 give both
    # projections a last tile column of 64 outputs and an odd number of
    # 64-wide K slices (65) for the two-stage ring.  The training forward
    # also keeps the GeLU input through the same path.
    w = inputs.Workload(23, "ragged_big_tile", "bf16", M=M, H=H, F=Fs, T=1)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    if train:
        Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
        U = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
        tp.tp_colpar_act_train(dev.X, dev.W1t, dev.b1, Y, U, M, H, Fs, 1, 0)
        Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(Y, dev.W2t, Z, M, H, Fs, 1, 0, tp.TP_BF16)
    else:
        Y, Z = dev.shard(1, 0, use_fused=False)
    torch.cuda.synchronize()
    rows = np.array([r for r in (0, 255, 256, 4095, 4096, 4150, 4195) if r < M])
    Yr, Zr = oracle.mlp_shard(X.f64[rows], W1.f64, b1.f64, W2.f64, 1, 0)
    ey, ez = rel_fro(to_f64(Y)[rows], Yr), rel_fro(to_f64(Z)[rows], Zr)
    print("  Y %.2e  Z %.2e" % (ey, ez))
    assert ey <= TOL["bf16"] and ez <= TOL["bf16"]
    if train:
        eu = rel_fro(to_f64(U)[rows], oracle.colpar_linear(X.f64[rows], W1.f64, b1.f64, 1, 0))
        print("  U %.2e" % eu)
        assert eu <= TOL["bf16"]


@pytest.mark.parametrize("M", [1800, 2600, 8192])
def test_rowpar_band_order_every_tile(M):
    # the row-parallel launch at H = 8192 on the 256 x 256 tile (32 tile
    # columns, four per XCD) takes the band tile order; 1800 tokens make one
    # group of 8 tile rows whose last is partial, 2600 a full group of 8 and
    # a group of 3.  One token row
    # per tile row and tile column pair (row r = 256 tm + (37 tm) % 256, every
    # column) is checked, so a tile the order skipped or computed twice fails
    H, Fs = 8192, 512
    w = inputs.Workload(44, "rowpar_bands", "bf16", M=M, H=H, F=Fs, T=1)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    Z = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    tp.tp_colpar_gelu(dev.X, dev.W1t, dev.b1, Y, M, H, Fs, 1, 0, tp.TP_BF16)
    tp.tp_rowpar_partial(Y, dev.W2t, Z, M, H, Fs, 1, 0, tp.TP_BF16)
    torch.cuda.synchronize()
    assert not torch.isnan(Z).any()
    tiles_m = (M + 255) // 256
    rows = np.array(sorted({min(M - 1, 256 * tm + (37 * tm) % 256) for tm in range(tiles_m)}))
    _, Zr = oracle.mlp_shard(X.f64[rows], W1.f64, b1.f64, W2.f64, 1, 0)
    Zg = to_f64(Z)[rows]
    for tn in range(H // 256):
        cols = slice(256 * tn, 256 * tn + 256)
        e = rel_fro(Zg[:, cols], Zr[:, cols])
        assert e <= TOL["bf16"], (tn, e)


@pytest.mark.parametrize("K", [64, 128, 192, 320, 448, 704])
def test_short_k_on_the_deep_b_ring(K):
    # the 256 x 256 forward tile keeps two A and three B stages and unrolls
    # six K slices; K = 64 .. 704 gives 1, 2, 3, 5, 7 and 11 slices, i.e.
    # prologues whose refills re-read the last slice and remainders of 1 to 5
    # slices after the unrolled loop.  Both launches run that tile here
    # (4096 x 4096 outputs: 256 tiles), the column-parallel one with K = H
    # and the row-parallel one with K = F/T.
    M, N = 4096, 4096
    wu = inputs.Workload(45, "short_k_up", "bf16", M=M, H=K, F=N, T=1)
    X, W1, b1, _ = inputs.mlp_inputs(wu)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tp.tp_colpar_gelu(X.torch(), W1.transposed().torch(), b1.torch(), Y, M, K, N, 1, 0, tp.TP_BF16)
    wd = inputs.Workload(46, "short_k_down", "bf16", M=M, H=N, F=K, T=1)
    Xd, _, _, W2 = inputs.mlp_inputs(wd)
    Yd = inputs.normal((M, K), 1.0, "bf16", workload=46, tensor=inputs.X_ID + 20)
    Z = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tp.tp_rowpar_partial(Yd.torch(), W2.transposed().torch(), Z, M, N, K, 1, 0, tp.TP_BF16)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 255, 256, 1000, 2047, 4095}))
    Yr = oracle.colpar_gelu(X.f64[rows], W1.f64, b1.f64, 1, 0)
    Zr = oracle.rowpar_partial(Yd.f64[rows], W2.f64, 1, 0)
    ey, ez = rel_fro(to_f64(Y)[rows], Yr), rel_fro(to_f64(Z)[rows], Zr)
    print("  K=%d: Y %.2e  Z %.2e" % (K, ey, ez))
    assert ey <= TOL["bf16"] and ez <= TOL["bf16"]


def test_full_matrix_and_rank_local_calls_agree_bitwise():
    # Shard i of the full W1^T/W2^T (F, T, i) is the same computation as the
    # stand-alone shard matrices (F/T, 1, 0); first and last shard.
    w = inputs.Workload(14, "bf16_t8", "bf16", M=96, H=256, F=8 * 128, T=8)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    Fs = w.F // 8
    for i in (0, 7):
        C = slice(i * Fs, (i + 1) * Fs)
        loc = DeviceMLP(X, inputs.Synth("bf16", np.ascontiguousarray(W1.data[:, C])),
                        inputs.Synth("bf16", np.ascontiguousarray(b1.data[C])),
                        inputs.Synth("bf16", np.ascontiguousarray(W2.data[C])))
        Yf, Zf = dev.shard(8, i)
        Yl, Zl = loc.shard(1, 0)
        torch.cuda.synchronize()
        assert torch.equal(Yf, Yl) and torch.equal(Zf, Zl)


# ----------------------------------------------------- bf16 decode path
@pytest.mark.parametrize("M", [1, 5, 16, 17, 32])
@pytest.mark.parametrize("H", [192, 768, 1024])
def test_decode_small(M, H):
    # H picks the K split of the weight-streaming kernel (1, 2 or 8 waves)
    w = inputs.Workload(15, "decode_small", "bf16", M=M, H=H, F=2 * 1024, T=2)
    check_all_shards(w, M=M, T=2)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_full_size_mlp_and_outproj(M):
    # H=8192, F/T=4096 MLP shard plus the attention out-projection shard
    # (8 heads x 128 = 1024 context dims per rank, W_o block [1024, 8192]).
    w = inputs.WORKLOADS["decode"]
    X, W1, b1, W2 = inputs.mlp_inputs(w, M=M, shard_only=0)
    dev = DeviceMLP(X, W1, b1, W2)
    Y, Z = dev.shard(1, 0)
    ctx, Wo = inputs.outproj_inputs(w, M=M, shard=0)
    dctx, dWot = ctx.torch(), Wo.transposed().torch()
    O = torch.empty(M, w.H, dtype=torch.float32, device="cuda")
    As = w.A // w.T
    tp.tp_rowpar_partial(dctx, dWot, O, M, w.H, As, 1, 0, tp.TP_BF16)
    torch.cuda.synchronize()
    Yr, Zr = oracle.mlp_shard(X.f64, W1.f64, b1.f64, W2.f64, 1, 0)
    Or = oracle.rowpar_partial(ctx.f64, Wo.f64, 1, 0)
    e = [rel_fro(to_f64(Y), Yr), rel_fro(to_f64(Z), Zr), rel_fro(to_f64(O), Or)]
    print("  Y_0 %.2e  Z_0 %.2e  O_0 %.2e" % tuple(e))
    assert max(e) <= TOL["bf16"]


@pytest.mark.parametrize("M", [17, 32])
def test_decode_two_token_tiles_full_width(M):
    # two token tiles (the token rows regrouped through LDS like the weights)
    # on a full-width rank share, H=8192, F/T=4096; M = 17 leaves the second
    # tile with a single token
    H, Fs = 8192, 4096
    w = inputs.Workload(24, "decode_two_tiles", "bf16", M=M, H=H, F=Fs, T=1)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    Y, Z = dev.shard(1, 0, use_fused=False)
    torch.cuda.synchronize()
    Yr, Zr = oracle.mlp_shard(X.f64, W1.f64, b1.f64, W2.f64, 1, 0)
    ey, ez = rel_fro(to_f64(Y), Yr), rel_fro(to_f64(Z), Zr)
    print("  Y %.2e  Z %.2e" % (ey, ez))
    assert ey <= TOL["bf16"] and ez <= TOL["bf16"]


def test_outproj_head_shards_sum_to_full_projection():
    # Head-sharded out-projection: T=8 ranks with the full W_o^T [H, A]; the
    # reduced partials equal ctx . W_o over all heads.
    H, A, T, M = 512, 1024, 8, 40
    ctx = inputs.normal((M, A), 1.0, "bf16", workload=16, tensor=inputs.CTX_ID)
    Wo = inputs.normal((A, H), 0.02, "bf16", workload=16, tensor=inputs.WO_ID)
    dctx, dWot = ctx.torch(), Wo.transposed().torch()
    parts = []
    for i in range(T):
        ci = dctx[:, i * A // T:(i + 1) * A // T].contiguous()
        O = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(ci, dWot, O, M, H, A, T, i, tp.TP_BF16)
        parts.append(O)
    out = torch.empty(M, H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce(parts, T, None, out, None, M, H)
    torch.cuda.synchronize()
    want = oracle.rowpar_partial(ctx.f64, Wo.f64, 1, 0)
    assert rel_fro(to_f64(out), want) <= TOL["bf16"]


# ------------------------------------------- whole-group (all shards) calls
def group_outputs(dev, T, split=False):
    Fs = dev.F // T
    tdt = torch.bfloat16 if dev.dt == "bf16" else torch.float32
    Ys = [torch.empty(dev.M, Fs, dtype=tdt, device="cuda") for _ in range(T)]
    Zs = [torch.empty(dev.M, dev.H, dtype=torch.float32, device="cuda") for _ in range(T)]
    dt = tp.TP_BF16 if dev.dt == "bf16" else tp.TP_F32
    if split:
        tp.tp_colpar_gelu_group(dev.X, dev.W1t, dev.b1, Ys, dev.M, dev.H, dev.F, T, dt)
        tp.tp_rowpar_partial_group(Ys, dev.W2t, Zs, dev.M, dev.H, dev.F, T, dt)
    else:
        tp.tp_mlp_group_fwd(dev.X, dev.W1t, dev.b1, dev.W2t, Ys, Zs, dev.M, dev.H, dev.F, T, dt)
    return Ys, Zs


@pytest.mark.parametrize("dt,M,H,F,T,split", [
    ("bf16", 300, 512, 1280, 4, False),    # MFMA GEMM, ragged M and N
    ("bf16", 2048, 1024, 4096, 4, True),   # enough tiles for the 256x256 config
    ("bf16", 8, 1024, 4096, 8, False),     # decode kernel, all 8 shards batched
    ("bf16", 32, 512, 2048, 2, True),
    ("f32", 40, 256, 1024, 2, False),
])
def test_group_matches_per_shard_calls_bitwise(dt, M, H, F, T, split):
    w = inputs.Workload(19, "group", dt, M=M, H=H, F=F, T=T)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    Ys, Zs = group_outputs(dev, T, split)
    per = [dev.shard(T, i) for i in range(T)]
    torch.cuda.synchronize()
    for i in range(T):
        assert torch.equal(Ys[i], per[i][0]) and torch.equal(Zs[i], per[i][1]), i
    rows = inputs.row_sample(M, 6)
    for i in (0, T - 1):
        Yr, Zr = oracle.mlp_shard(X.f64[rows], W1.f64, b1.f64, W2.f64, T, i)
        assert rel_fro(to_f64(Ys[i])[rows], Yr) <= TOL[dt] and rel_fro(to_f64(Zs[i])[rows], Zr) <= TOL[dt]


def test_group_gpt_block_shard_full_size():
    # the benchmarked launch: H=4096, F=16384, T=4, M=2048, all shards in one
    # launch per projection, then the reduce; sampled rows against the oracle
    w = inputs.WORKLOADS["gpt_block_shard"]
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    Ys, Zs = group_outputs(dev, w.T)
    Z = torch.empty(w.M, w.H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce(Zs, w.T, None, Z, None, w.M, w.H)
    torch.cuda.synchronize()
    rows = inputs.row_sample(w.M, 10, seed=5)
    _, Zu = oracle.mlp_unsharded(X.f64[rows], W1.f64, b1.f64, W2.f64)
    e = rel_fro(to_f64(Z)[rows], Zu)
    print("  reduced Z vs unsharded oracle: %.2e" % e)
    assert e <= TOL["bf16"]


# ------------------------------------------------------------- reduce
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_reduce_integer_partials_exact(T):
    M, H = 37, 256
    g = torch.Generator().manual_seed(T)
    P = [torch.randint(-1000, 1000, (M, H), generator=g).float().cuda() for _ in range(T)]
    R = torch.randint(-1000, 1000, (M, H), generator=g).float().cuda()
    out = torch.empty(M, H, device="cuda")
    tp.tp_shard_reduce(P, T, R, out, None, M, H)
    want = oracle.shard_reduce(np.stack([to_f64(p) for p in P]), to_f64(R))
    assert np.array_equal(to_f64(out), want)
    # in place on the residual stream
    tp.tp_shard_reduce(P, T, R, R, None, M, H)
    assert np.array_equal(to_f64(R), want)


def test_reduce_bf16_copy_is_round_to_nearest_even():
    M, H, T = 64, 1024, 4
    g = torch.Generator().manual_seed(5)
    P = [torch.randn(M, H, generator=g).cuda() * 3 for _ in range(T)]
    out = torch.empty(M, H, device="cuda")
    ob = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    tp.tp_shard_reduce(P, T, None, out, ob, M, H)
    host = out.cpu().numpy()
    assert np.array_equal(ob.cpu().view(torch.int16).numpy().view(np.uint16), inputs.f32_to_bf16_bits(host))


def test_reduce_bf16_copy_ties_subnormals_and_specials():
    # one partial (the sum is the value itself): exact ties between two bf16
    # neighbours go to the even one, subnormals round like normals, infinities
    # stay, NaNs stay NaN; the device's conversion against the host RNE
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000, 0x7F7F8000, 0x7F7FFFFF],
                    dtype=np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38, -3.4e38, 1.5e-45], dtype=np.float32)
    vals = np.concatenate([ties, special])
    M, H = 2, 64
    x = np.zeros((M, H), dtype=np.float32)
    x.flat[:len(vals)] = vals
    x[1, :] = np.nan
    P = torch.from_numpy(x).cuda()
    out = torch.empty(M, H, device="cuda")
    ob = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    tp.tp_shard_reduce([P], 1, None, out, ob, M, H)
    torch.cuda.synchronize()
    got = ob.cpu().view(torch.int16).numpy().view(np.uint16)
    want = inputs.f32_to_bf16_bits(x)
    assert np.array_equal(got[0], want[0]), [hex(v) for v in got[0][:len(vals)]]
    assert np.isnan(inputs.bf16_bits_to_f32(got[1])).all()


# the row-RMS kernel runs 1024 threads per row, two 16-byte elements per
# thread and pass: H = 64 leaves most threads idle, 4160 gives a ragged second
# element, 8192 is exactly one pass, 12288 two passes; in place is how the
# layer driver calls it (the sum overwrites the residual)
@pytest.mark.parametrize("H,inplace", [(64, False), (4160, False), (8192, False), (12288, False), (12288, True)])
def test_reduce_rms_copy(H, inplace):
    M, T = 9, 8
    g = torch.Generator().manual_seed(H)
    P = [torch.randn(M, H, generator=g).cuda() * 50 for _ in range(T)]
    R = torch.randn(M, H, generator=g).cuda()
    want, wrms = oracle.shard_reduce(np.stack([to_f64(p) for p in P]), to_f64(R), rms_eps=tp.TP_RMS_EPS)
    out = R if inplace else torch.empty(M, H, device="cuda")
    ob = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    tp.tp_shard_reduce(P, T, R, out, ob, M, H, tp.TP_REDUCE_RMS_BF16)
    assert rel_fro(to_f64(out), want) <= 1e-6
    assert rel_fro(to_f64(ob), wrms) <= TOL["bf16"]


# partials larger than half the last-level cache (the 80-layer stack's
# prefill reduces) are read with streaming loads: the same sums, exactly, in
# place on the residual stream as the layer driver calls it, with and without
# the row-RMS copy (ragged rows and a ragged last pass of the RMS kernel)
@pytest.mark.parametrize("rms", [False, True])
def test_reduce_streamed_partials(rms):
    M, H, T = 1100, 4100, 8
    assert T * M * H * 4 > 128 << 20
    g = torch.Generator().manual_seed(11)
    P = [torch.randint(-1000, 1000, (M, H), generator=g).float().cuda() for _ in range(T)]
    R = torch.randint(-1000, 1000, (M, H), generator=g).float().cuda()
    parts = np.stack([to_f64(p) for p in P])
    ob = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    if rms:
        want, wrms = oracle.shard_reduce(parts, to_f64(R), rms_eps=tp.TP_RMS_EPS)
        tp.tp_shard_reduce(P, T, R, R, ob, M, H, tp.TP_REDUCE_RMS_BF16)
        assert rel_fro(to_f64(ob), wrms) <= TOL["bf16"]
    else:
        want = oracle.shard_reduce(parts, to_f64(R))
        tp.tp_shard_reduce(P, T, R, R, None, M, H)
    assert np.array_equal(to_f64(R), want)


# -------------------------------------------------------- edge cases
def test_empty_call_touches_nothing():
    X = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(128, 64, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_colpar_gelu(X, W, None, Y, 0, 64, 128, 2, 1, tp.TP_BF16)
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())


@pytest.mark.parametrize("M", [8, 300])
def test_nan_in_one_row_stays_in_that_row(M):
    w = inputs.Workload(17, "nan_row", "bf16", M=M, H=256, F=512, T=2)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    X.data[3, 17] = 0x7FC0  # bf16 quiet NaN
    dev = DeviceMLP(X, W1, b1, W2)
    _, Z = dev.all_shards_reduced(2)
    torch.cuda.synchronize()
    bad = torch.isnan(Z).any(dim=1).cpu().numpy()
    assert bad[3] and bad.sum() == 1


@pytest.mark.parametrize("M", [8, 520])
def test_runs_are_bitwise_deterministic(M):
    w = inputs.Workload(18, "determinism", "bf16", M=M, H=1024, F=4096, T=4)
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dev = DeviceMLP(X, W1, b1, W2)
    _, Z1 = dev.all_shards_reduced(4)
    _, Z2 = dev.all_shards_reduced(4)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)


def test_gelu_epilogue_accuracy_dense_grid():
    # fp32 mode with W1 = [I | 0]: Y_i is GeLU evaluated on the exact inputs.
    H = 64
    x = np.linspace(-12, 12, 64 * 1024).astype(np.float32)
    M = x.size // H
    X = x.reshape(M, H)
    W1 = np.eye(H, dtype=np.float32)
    dX = torch.from_numpy(X).cuda()
    dW1t = torch.from_numpy(np.ascontiguousarray(W1.T)).cuda()
    Y = torch.empty(M, H, device="cuda")
    tp.tp_colpar_gelu(dX, dW1t, None, Y, M, H, H, 1, 0, tp.TP_F32)
    torch.cuda.synchronize()
    want = oracle.gelu(X.astype(np.float64))
    err = np.abs(Y.cpu().numpy().astype(np.float64) - want)
    assert np.max(err / (1 + np.abs(want))) <= 2e-6
