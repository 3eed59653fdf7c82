"""The backward pass of a rank's MLP share through the C ABI against the fp64
oracle: the training forward that keeps the GeLU input, the row-parallel
backward (input gradient fused with GeLU', weight gradient), the column-
parallel backward (input-gradient partial, weight and bias gradients), the
accumulate mode, the whole TP group's backward with the dX partials reduced
on device against the unsharded gradients, and the full-size rank shape on
sampled gradient columns and rows."""
import sys

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colpar_amd import inputs
from tests.harness import TOL, rel_fro, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from megatron_tensor_transformer_colpar_amd import tp

TANH, ERF = oracle.ACT_GELU_TANH, oracle.ACT_GELU_ERF
DZ_ID = 30


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def act_code(form):
    return tp.TP_GELU_ERF if form == ERF else tp.TP_GELU_TANH


class Problem:
    """Seeded inputs of one MLP block and its output gradient, on host and GPU."""

    def __init__(self, wid, M, H, F, T, form=TANH, dz_std=1.0):
        w = inputs.Workload(wid, "bwd", "bf16", M=M, H=H, F=F, T=T)
        self.X, self.W1, self.b1, self.W2 = inputs.mlp_inputs(w, M=M)
        self.dZ = inputs.normal((M, H), dz_std, "bf16", seed=0, workload=wid, tensor=DZ_ID)
        self.M, self.H, self.F, self.T, self.Fs = M, H, F, T, F // T
        self.form = form
        self.dX_, self.dW1t, self.db1 = self.X.torch(), self.W1.transposed().torch(), self.b1.torch()
        self.dW2t, self.ddZ = self.W2.transposed().torch(), self.dZ.torch()

    def oracle(self, T=None, i=0):
        return oracle.mlp_shard_bwd(self.X.f64, self.W1.f64, self.b1.f64, self.W2.f64, self.dZ.f64,
                                    self.T if T is None else T, i, self.form)

    def forward_train(self, i):
        Y = torch.empty(self.M, self.Fs, dtype=torch.bfloat16, device="cuda")
        U = torch.empty_like(Y)
        tp.tp_colpar_act_train(self.dX_, self.dW1t, self.db1, Y, U, self.M, self.H, self.F, self.T, i,
                               act_code(self.form))
        return Y, U


@pytest.mark.parametrize("M,form", [(300, TANH), (8, ERF), (1, TANH)])
def test_forward_train_keeps_the_gelu_input(M, form):
    p = Problem(70, M, 512, 2048, 2, form)
    for i in range(2):
        Y, U = p.forward_train(i)
        torch.cuda.synchronize()
        eu = rel_fro(to_f64(U), oracle.colpar_linear(p.X.f64, p.W1.f64, p.b1.f64, 2, i))
        ey = rel_fro(to_f64(Y), oracle.colpar_act(p.X.f64, p.W1.f64, p.b1.f64, 2, i, form))
        print("  rank %d: U %.2e Y %.2e" % (i, eu, ey))
        assert max(eu, ey) <= TOL["bf16"]


@pytest.mark.parametrize("M,H,F,T,form", [
    (256, 512, 2048, 2, TANH),      # 256x128 tiles
    (300, 512, 2048, 2, ERF),       # ragged tokens (K of the weight gradient is ragged)
    (8, 1024, 2048, 2, TANH),       # decode-sized: one 64-token slice of K
    (2048, 1024, 4096, 2, TANH),    # 256x256 tiles for the weight gradient
])
def test_rowpar_bwd(M, H, F, T, form):
    p = Problem(71, M, H, F, T, form)
    for i in range(T):
        Y, U = p.forward_train(i)
        dU = torch.empty_like(Y)
        dW2t = torch.zeros(H, F, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_bwd(p.ddZ, p.dW2t, Y, U, dU, dW2t, M, H, F, T, i, act_code(form))
        torch.cuda.synchronize()
        o = p.oracle(i=i)
        Fs = F // T
        e = (rel_fro(to_f64(dU), o["dU_i"]), rel_fro(to_f64(dW2t[:, i * Fs:(i + 1) * Fs]).T, o["dW2_i"]))
        print("  rank %d: dU %.2e dW2 %.2e" % (i, e[0], e[1]))
        assert max(e) <= TOL["bf16"]
        other = torch.cat([dW2t[:, :i * Fs], dW2t[:, (i + 1) * Fs:]], dim=1)
        assert not bool(other.any()), "wrote outside rank i's columns of dW2^T"


def test_rowpar_bwd_without_activation_is_the_plain_input_gradient():
    # the head-sharded out-projection's backward: dctx_i = dO . W_o[A_i, :]^T
    M, H, A, T = 96, 512, 1024, 2
    p = Problem(72, M, H, A, T)
    i = 1
    As = A // T
    ctx = inputs.normal((M, As), 1.0, "bf16", seed=0, workload=72, tensor=inputs.CTX_ID)
    dctx = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
    dWot = torch.zeros(H, A, dtype=torch.float32, device="cuda")
    tp.tp_rowpar_bwd(p.ddZ, p.dW2t, ctx.torch(), None, dctx, dWot, M, H, A, T, i)
    torch.cuda.synchronize()
    want = p.dZ.f64 @ p.W2.f64[i * As:(i + 1) * As].T
    wantW = (ctx.f64.T @ p.dZ.f64).T
    e = (rel_fro(to_f64(dctx), want), rel_fro(to_f64(dWot[:, i * As:]), wantW))
    print("  dctx %.2e dWo %.2e" % e)
    assert max(e) <= TOL["bf16"]


@pytest.mark.parametrize("M,H,F,T,form", [
    (256, 512, 2048, 2, TANH),
    (300, 512, 2048, 2, ERF),
    (8, 1024, 2048, 2, TANH),
    (2048, 1024, 4096, 2, TANH),
])
def test_colpar_bwd(M, H, F, T, form):
    p = Problem(73, M, H, F, T, form)
    Fs = F // T
    for i in range(T):
        o = p.oracle(i=i)
        dU = inputs.from_values(o["dU_i"], "bf16")   # the oracle's GeLU-input gradient, rounded
        dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
        dW1t = torch.zeros(F, H, dtype=torch.float32, device="cuda")
        db1 = torch.zeros(F, dtype=torch.float32, device="cuda")
        tp.tp_colpar_bwd(p.dX_, p.dW1t, dU.torch(), dX, dW1t, db1, M, H, F, T, i)
        torch.cuda.synchronize()
        W1i = p.W1.f64[:, i * Fs:(i + 1) * Fs]
        e = (rel_fro(to_f64(dX), dU.f64 @ W1i.T), rel_fro(to_f64(dW1t[i * Fs:(i + 1) * Fs]).T, p.X.f64.T @ dU.f64),
             rel_fro(to_f64(db1[i * Fs:(i + 1) * Fs]), dU.f64.sum(axis=0)))
        print("  rank %d: dX %.2e dW1 %.2e db1 %.2e" % (i, *e))
        assert max(e) <= TOL["bf16"]
        # and against the oracle's own gradients (the rounding of dU included)
        e2 = (rel_fro(to_f64(dX), o["dX_i"]), rel_fro(to_f64(dW1t[i * Fs:(i + 1) * Fs]).T, o["dW1_i"]))
        assert max(e2) <= TOL["bf16"]
        assert not bool(torch.cat([dW1t[:i * Fs], dW1t[(i + 1) * Fs:]]).any())


def test_gradients_accumulate_and_optional_outputs():
    M, H, F, T = 128, 512, 1024, 2
    p = Problem(74, M, H, F, T)
    i, Fs = 0, F // T
    Y, U = p.forward_train(i)
    dU = torch.empty_like(Y)
    base = torch.randn(H, F, device="cuda")
    dW2t = base.clone()
    tp.tp_rowpar_bwd(p.ddZ, p.dW2t, Y, U, dU, dW2t, M, H, F, T, i, flags=tp.TP_GRAD_ACCUMULATE)
    dW1t = torch.randn(F, H, device="cuda")
    db1 = torch.randn(F, device="cuda")
    dW1t0, db10 = dW1t.clone(), db1.clone()
    tp.tp_colpar_bwd(p.dX_, None, dU, None, dW1t, db1, M, H, F, T, i, flags=tp.TP_GRAD_ACCUMULATE)
    torch.cuda.synchronize()
    o = p.oracle(i=i)
    e = (rel_fro(to_f64(dW2t - base)[:, :Fs].T, o["dW2_i"]), rel_fro(to_f64(dW1t - dW1t0)[:Fs].T, o["dW1_i"]),
         rel_fro(to_f64(db1 - db10)[:Fs], o["db1_i"]))
    print("  accumulated dW2 %.2e dW1 %.2e db1 %.2e" % e)
    assert max(e) <= TOL["bf16"]
    assert torch.equal(dW2t[:, Fs:], base[:, Fs:]) and torch.equal(db1[Fs:], db10[Fs:])
    # only the input gradient
    dU2 = torch.empty_like(Y)
    tp.tp_rowpar_bwd(p.ddZ, p.dW2t, None, U, dU2, None, M, H, F, T, i)
    torch.cuda.synchronize()
    assert torch.equal(dU2, dU)


@pytest.mark.parametrize("T", [2, 4])
def test_group_backward_reassembles_the_unsharded_gradients(T):
    # every rank's forward and backward; the dX partials summed on device (the
    # backward all-reduce), the weight-gradient blocks of all ranks together
    M, H, F = 200, 512, 2048
    p = Problem(75, M, H, F, T, ERF)
    Fs = F // T
    dW1t = torch.zeros(F, H, dtype=torch.float32, device="cuda")
    db1 = torch.zeros(F, dtype=torch.float32, device="cuda")
    dW2t = torch.zeros(H, F, dtype=torch.float32, device="cuda")
    dXs = []
    for i in range(T):
        Y, U = p.forward_train(i)
        dU = torch.empty_like(Y)
        dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tp.tp_mlp_shard_bwd(p.dX_, p.dW1t, p.dW2t, U, Y, p.ddZ, dU, dX, dW1t, db1, dW2t, M, H, F, T, i,
                            act_code(ERF))
        dXs.append(dX)
    dXsum = torch.empty(M, H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce(dXs, T, None, dXsum, None, M, H)
    torch.cuda.synchronize()
    o = p.oracle(T=1, i=0)
    e = (rel_fro(to_f64(dXsum), o["dX_i"]), rel_fro(to_f64(dW1t).T, o["dW1_i"]), rel_fro(to_f64(db1), o["db1_i"]),
         rel_fro(to_f64(dW2t).T, o["dW2_i"]))
    print("  dX %.2e dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]


def test_backward_full_size_sampled():
    # rank 1 of the 2048-token block (H=4096, F=16384, T=4) on its own weight
    # blocks: sampled gradient columns are exact on their own (each column's
    # gradients involve only that column), sampled dX rows likewise
    w = inputs.WORKLOADS["gpt_block_shard"]
    M, H, Fs = w.M, w.H, w.F // w.T
    X, W1, b1, W2 = inputs.mlp_inputs(w, shard_only=1)
    dZ = inputs.normal((M, H), 1.0, "bf16", seed=0, workload=w.wid, tensor=DZ_ID)
    dX_, dW1t_, db1_, dW2t_ = X.torch(), W1.transposed().torch(), b1.torch(), W2.transposed().torch()
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    U = torch.empty_like(Y)
    dU = torch.empty_like(Y)
    dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
    dW1t = torch.empty(Fs, H, dtype=torch.float32, device="cuda")
    db1 = torch.empty(Fs, dtype=torch.float32, device="cuda")
    dW2t = torch.empty(H, Fs, dtype=torch.float32, device="cuda")
    tp.tp_colpar_act_train(dX_, dW1t_, db1_, Y, U, M, H, Fs, 1, 0)
    tp.tp_mlp_shard_bwd(dX_, dW1t_, dW2t_, U, Y, dZ.torch(), dU, dX, dW1t, db1, dW2t, M, H, Fs, 1, 0)
    torch.cuda.synchronize()
    cols = inputs.row_sample(Fs, 12, seed=3)
    oc = oracle.mlp_shard_bwd(X.f64, W1.f64[:, cols], b1.f64[cols], W2.f64[cols], dZ.f64, 1, 0)
    e = (rel_fro(to_f64(dU)[:, cols], oc["dU_i"]), rel_fro(to_f64(dW1t)[cols].T, oc["dW1_i"]),
         rel_fro(to_f64(db1)[cols], oc["db1_i"]), rel_fro(to_f64(dW2t)[:, cols].T, oc["dW2_i"]))
    print("  columns: dU %.2e dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]
    rows = inputs.row_sample(M, 24, seed=4)
    orow = oracle.mlp_shard_bwd(X.f64[rows], W1.f64, b1.f64, W2.f64, dZ.f64[rows], 1, 0)
    er = rel_fro(to_f64(dX)[rows], orow["dX_i"])
    print("  rows: dX %.2e" % er)
    assert er <= TOL["bf16"]


def test_backward_prefill_rank_shape_sampled():
    # rank 0 of the pages' prefill shape (H=8192, F/T=4096, M=8192), as the
    # bench times it: every launch on 256x256 tiles, dU and dX on 16x16x32
    # transpose-read fragments, dW1 and dW2 on 32x32x16; sampled gradient
    # columns (first and last included) and sampled dX rows against the oracle
    w = inputs.WORKLOADS["prefill"]
    M, H, Fs = w.M, w.H, w.F // w.T
    X, W1, b1, W2 = inputs.mlp_inputs(w, shard_only=0)
    dZ = inputs.normal((M, H), 1.0, "bf16", seed=0, workload=w.wid, tensor=DZ_ID)
    dX_, dW1t_, db1_, dW2t_ = X.torch(), W1.transposed().torch(), b1.torch(), W2.transposed().torch()
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    U = torch.empty_like(Y)
    dU = torch.empty_like(Y)
    dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
    dW1t = torch.empty(Fs, H, dtype=torch.float32, device="cuda")
    db1 = torch.empty(Fs, dtype=torch.float32, device="cuda")
    dW2t = torch.empty(H, Fs, dtype=torch.float32, device="cuda")
    tp.tp_colpar_act_train(dX_, dW1t_, db1_, Y, U, M, H, Fs, 1, 0)
    tp.tp_mlp_shard_bwd(dX_, dW1t_, dW2t_, U, Y, dZ.torch(), dU, dX, dW1t, db1, dW2t, M, H, Fs, 1, 0)
    torch.cuda.synchronize()
    cols = inputs.row_sample(Fs, 8, seed=5)
    oc = oracle.mlp_shard_bwd(X.f64, W1.f64[:, cols], b1.f64[cols], W2.f64[cols], dZ.f64, 1, 0)
    e = (rel_fro(to_f64(dU)[:, cols], oc["dU_i"]), rel_fro(to_f64(dW1t)[cols].T, oc["dW1_i"]),
         rel_fro(to_f64(db1)[cols], oc["db1_i"]), rel_fro(to_f64(dW2t)[:, cols].T, oc["dW2_i"]))
    print("  columns: dU %.2e dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]
    rows = inputs.row_sample(M, 16, seed=6)
    orow = oracle.mlp_shard_bwd(X.f64[rows], W1.f64, b1.f64, W2.f64, dZ.f64[rows], 1, 0)
    er = rel_fro(to_f64(dX)[rows], orow["dX_i"])
    print("  rows: dX %.2e" % er)
    assert er <= TOL["bf16"]


def test_weight_gradients_on_256x128_tiles():
    # H=4096, F/T=2048: the weight gradients (2048 x 4096 and 4096 x 2048)
    # are 128 tiles of 256x256 but 256 of 256x128, so they take the 256x128
    # tile (two B fragments per wave, single-buffered); 520 tokens make their
    # K ragged (8 slices of 64 and 8 left over); sampled gradient columns,
    # exact on their own, against the oracle
    M, H, F, T = 520, 4096, 4096, 2
    p = Problem(77, M, H, F, T, ERF)
    Fs = p.Fs
    i = 1
    Y, U = p.forward_train(i)
    dU = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
    # the full gradients: rank i writes its block (rows C_i of dW1^T, entries
    # C_i of db1, columns C_i of dW2^T)
    dW1t = torch.zeros(F, H, dtype=torch.float32, device="cuda")
    db1 = torch.zeros(F, dtype=torch.float32, device="cuda")
    dW2t = torch.zeros(H, F, dtype=torch.float32, device="cuda")
    tp.tp_mlp_shard_bwd(p.dX_, p.dW1t, p.dW2t, U, Y, p.ddZ, dU, dX, dW1t, db1, dW2t, M, H, F, T, i,
                        act_code(ERF))
    torch.cuda.synchronize()
    cols = inputs.row_sample(Fs, 12, seed=7)
    gcols = i * Fs + cols
    oc = oracle.mlp_shard_bwd(p.X.f64, p.W1.f64[:, gcols], p.b1.f64[gcols], p.W2.f64[gcols], p.dZ.f64, 1, 0, ERF)
    e = (rel_fro(to_f64(dU)[:, cols], oc["dU_i"]), rel_fro(to_f64(dW1t)[gcols].T, oc["dW1_i"]),
         rel_fro(to_f64(db1)[gcols], oc["db1_i"]), rel_fro(to_f64(dW2t)[:, gcols].T, oc["dW2_i"]))
    print("  columns: dU %.2e dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]


@pytest.mark.parametrize("F", [8192, 4096])
def test_weight_gradients_accumulate_on_large_tiles(F):
    # H=4096, T=2: F/T = 4096 makes the weight gradients 256 tiles of
    # 256x256, F/T = 2048 makes them 256 of 256x128; 520 tokens make their K
    # ragged.  Accumulating into random gradients: the increments of rank i's
    # sampled columns against the oracle, everything outside rank i's blocks
    # untouched
    M, H, T = 520, 4096, 2
    p = Problem(78, M, H, F, T)
    Fs = p.Fs
    i = 1
    Y, U = p.forward_train(i)
    dU = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    dW1t0 = torch.randn(F, H, generator=g, device="cuda")
    db10 = torch.randn(F, generator=g, device="cuda")
    dW2t0 = torch.randn(H, F, generator=g, device="cuda")
    dW1t, db1, dW2t = dW1t0.clone(), db10.clone(), dW2t0.clone()
    tp.tp_mlp_shard_bwd(p.dX_, p.dW1t, p.dW2t, U, Y, p.ddZ, dU, dX, dW1t, db1, dW2t, M, H, F, T, i,
                        flags=tp.TP_GRAD_ACCUMULATE)
    torch.cuda.synchronize()
    cols = inputs.row_sample(Fs, 12, seed=9)
    gcols = i * Fs + cols
    oc = oracle.mlp_shard_bwd(p.X.f64, p.W1.f64[:, gcols], p.b1.f64[gcols], p.W2.f64[gcols], p.dZ.f64, 1, 0)
    e = (rel_fro(to_f64(dW1t - dW1t0)[gcols].T, oc["dW1_i"]), rel_fro(to_f64(db1 - db10)[gcols], oc["db1_i"]),
         rel_fro(to_f64(dW2t - dW2t0)[:, gcols].T, oc["dW2_i"]))
    print("  accumulated columns: dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]
    assert torch.equal(dW1t[:i * Fs], dW1t0[:i * Fs]) and torch.equal(db1[:i * Fs], db10[:i * Fs])
    assert torch.equal(dW2t[:, :i * Fs], dW2t0[:, :i * Fs])


@pytest.mark.parametrize("T,M", [(4, 256), (2, 130)])
def test_group_entry_points(T, M):
    # the whole group's training forward and backward, one launch per
    # projection: against the unsharded oracle gradients and the per-rank calls
    H, F = 512, 2048
    p = Problem(76, M, H, F, T, TANH)
    Fs = F // T
    bf = lambda: torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    Ys, Us, dUs = [bf() for _ in range(T)], [bf() for _ in range(T)], [bf() for _ in range(T)]
    dXs = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]
    dW1t = torch.empty(F, H, dtype=torch.float32, device="cuda")
    db1 = torch.empty(F, dtype=torch.float32, device="cuda")
    dW2t = torch.empty(H, F, dtype=torch.float32, device="cuda")
    tp.tp_mlp_group_fwd_train(p.dX_, p.dW1t, p.db1, Ys, Us, M, H, F, T)
    tp.tp_mlp_group_bwd(p.dX_, p.dW1t, p.dW2t, Us, Ys, p.ddZ, dUs, dXs, dW1t, db1, dW2t, M, H, F, T)
    dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce(dXs, T, None, dX, None, M, H)
    torch.cuda.synchronize()
    o = p.oracle(T=1, i=0)
    e = (rel_fro(to_f64(dX), o["dX_i"]), rel_fro(to_f64(dW1t).T, o["dW1_i"]), rel_fro(to_f64(db1), o["db1_i"]),
         rel_fro(to_f64(dW2t).T, o["dW2_i"]))
    print("  dX %.2e dW1 %.2e db1 %.2e dW2 %.2e" % e)
    assert max(e) <= TOL["bf16"]
    # the per-rank entry points give the same numbers
    for i in (0, T - 1):
        Y, U = p.forward_train(i)
        dU = torch.empty_like(Y)
        dXi = torch.empty(M, H, dtype=torch.float32, device="cuda")
        w1 = torch.empty(F, H, dtype=torch.float32, device="cuda")
        b = torch.empty(F, dtype=torch.float32, device="cuda")
        w2 = torch.empty(H, F, dtype=torch.float32, device="cuda")
        tp.tp_mlp_shard_bwd(p.dX_, p.dW1t, p.dW2t, U, Y, p.ddZ, dU, dXi, w1, b, w2, M, H, F, T, i)
        torch.cuda.synchronize()
        sl = slice(i * Fs, (i + 1) * Fs)
        assert torch.equal(Y, Ys[i]) and torch.equal(U, Us[i])
        d = max(rel_fro(to_f64(dU), to_f64(dUs[i])), rel_fro(to_f64(dXi), to_f64(dXs[i])),
                rel_fro(to_f64(w1[sl]), to_f64(dW1t[sl])), rel_fro(to_f64(w2[:, sl]), to_f64(dW2t[:, sl])),
                rel_fro(to_f64(b[sl]), to_f64(db1[sl])))
        print("  rank %d: group vs per-rank %.1e" % (i, d))
        assert d <= 1e-6
