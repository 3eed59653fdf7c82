"""The exact GeLU form (tp_colpar_act) and the gated Gate/Up first layer
(tp_colpar_gated) through the C ABI against the fp64 oracle, on every kernel
path: the prefill GEMM (both gated tile shapes), the two skinny-M stream
kernels, the fp32 path; ragged token counts, with and without biases, and
the full-size shapes on sampled rows."""
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

ERF, TANH = oracle.ACT_GELU_ERF, oracle.ACT_GELU_TANH


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


def act_code(form):
    return tp.TP_GELU_ERF if form == ERF else tp.TP_GELU_TANH


# ------------------------------------------------------------ exact GeLU
@pytest.mark.parametrize("M,H,F,T,dt", [
    (33, 256, 1024, 2, "bf16"),     # prefill GEMM, ragged M
    (300, 512, 2048, 4, "bf16"),    # prefill GEMM, several tiles
    (1, 192, 2048, 2, "bf16"),      # skinny-M, 16-rows-x-64-bytes kernel
    (17, 1024, 2048, 2, "bf16"),    # skinny-M, segmented kernel, two token tiles
    (8, 256, 1024, 2, "f32"),       # fp32 path
])
def test_colpar_act_erf(M, H, F, T, dt):
    w = inputs.Workload(50, "act_erf", dt, M=M, H=H, F=F, T=T)
    X, W1, b1, _ = inputs.mlp_inputs(w, M=M)
    dX, dW1t, db1 = X.torch(), W1.transposed().torch(), b1.torch()
    i = T - 1
    Y = torch.empty(M, F // T, dtype=torch_dtype(dt), device="cuda")
    tp.tp_colpar_act(dX, dW1t, db1, Y, M, H, F, T, i, tp.TP_GELU_ERF, dtcode(dt))
    torch.cuda.synchronize()
    e = rel_fro(to_f64(Y), oracle.colpar_act(X.f64, W1.f64, b1.f64, T, i, ERF))
    print("  Y_%d %.2e" % (i, e))
    assert e <= TOL[dt]


@pytest.mark.parametrize("M", [8, 40])
def test_colpar_act_tanh_is_colpar_gelu(M):
    w = inputs.Workload(51, "act_tanh", "bf16", M=M, H=1024, F=2048, T=2)
    X, W1, b1, _ = inputs.mlp_inputs(w, M=M)
    dX, dW1t, db1 = X.torch(), W1.transposed().torch(), b1.torch()
    Ya = torch.empty(M, 1024, dtype=torch.bfloat16, device="cuda")
    Yg = torch.empty_like(Ya)
    tp.tp_colpar_act(dX, dW1t, db1, Ya, M, 1024, 2048, 2, 1, tp.TP_GELU_TANH)
    tp.tp_colpar_gelu(dX, dW1t, db1, Yg, M, 1024, 2048, 2, 1, tp.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yg)


# ------------------------------------------------------- gated first layer
def run_gated(X, Wg, Wu, bg, bu, M, H, F, T, i, form, dt):
    Y = torch.empty(M, F // T, dtype=torch_dtype(dt), device="cuda")
    tp.tp_colpar_gated(X.torch(), Wg.transposed().torch(), Wu.transposed().torch(),
                       None if bg is None else bg.torch(), None if bu is None else bu.torch(),
                       Y, M, H, F, T, i, act_code(form), dtcode(dt))
    return Y


@pytest.mark.parametrize("form", [TANH, ERF])
@pytest.mark.parametrize("M,H,F,T,bias,dt", [
    (64, 512, 2048, 2, True, "bf16"),     # prefill GEMM, 128x128 tiles
    (300, 512, 2048, 2, False, "bf16"),   # ragged M, no biases
    (1, 192, 2048, 2, True, "bf16"),      # skinny-M, 16-rows-x-64-bytes kernel
    (8, 1024, 2048, 2, False, "bf16"),    # skinny-M, segmented, 4 waves per block
    (17, 1024, 4096, 2, True, "bf16"),    # segmented, two token tiles
    (32, 768, 2048, 2, True, "bf16"),     # segmented, one wave per block
    (8, 256, 1024, 2, True, "f32"),       # fp32 path
])
def test_gated(form, M, H, F, T, bias, dt):
    w = inputs.Workload(52, "gated_small", dt, M=M, H=H, F=F, T=T)
    X, Wg, Wu, bg, bu = inputs.gated_inputs(w, M=M)
    if not bias:
        bg = bu = None
    for i in range(T):
        Y = run_gated(X, Wg, Wu, bg, bu, M, H, F, T, i, form, dt)
        torch.cuda.synchronize()
        want = oracle.colpar_gated(X.f64, Wg.f64, Wu.f64, None if bg is None else bg.f64,
                                   None if bu is None else bu.f64, T, i, form)
        e = rel_fro(to_f64(Y), want)
        print("  Y_%d %.2e" % (i, e))
        assert e <= TOL[dt]


def test_gated_prefill_full_size_sampled_rows():
    # rank 1 of the 2048-token block (H=4096, F=16384, T=4) on its own weight
    # blocks: 8 x 32 tiles of 256 rows x 128 output columns, then the
    # row-parallel partial of the gated activation
    w = inputs.WORKLOADS["gpt_block_shard"]
    M, H, Fs = w.M, w.H, w.F // w.T
    X, Wg, Wu, bg, bu = inputs.gated_inputs(w, shard_only=1)
    _, _, _, W2 = inputs.mlp_inputs(w, shard_only=1)
    for form in (TANH, ERF):
        Y = run_gated(X, Wg, Wu, bg, bu, M, H, Fs, 1, 0, form, "bf16")
        Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(Y, W2.transposed().torch(), Z, M, H, Fs, 1, 0, tp.TP_BF16)
        torch.cuda.synchronize()
        rows = inputs.row_sample(M, 48, seed=5)
        Yr = oracle.colpar_gated(X.f64[rows], Wg.f64, Wu.f64, bg.f64, bu.f64, 1, 0, form)
        Zr = oracle.rowpar_partial(Yr, W2.f64, 1, 0)
        e = (rel_fro(to_f64(Y)[rows], Yr), rel_fro(to_f64(Z)[rows], Zr))
        print("  form %d: Y %.2e  Z %.2e" % (form, e[0], e[1]))
        assert max(e) <= TOL["bf16"]


@pytest.mark.parametrize("M", [1, 8, 32])
def test_gated_decode_full_size(M):
    # rank 0 at H=8192, F/T=4096: every token row against the oracle
    w = inputs.WORKLOADS["decode"]
    X, Wg, Wu, bg, bu = inputs.gated_inputs(w, M=M, shard_only=0)
    Fs = w.F // w.T
    Y = run_gated(X, Wg, Wu, bg, bu, M, w.H, Fs, 1, 0, ERF, "bf16")
    torch.cuda.synchronize()
    e = rel_fro(to_f64(Y), oracle.colpar_gated(X.f64, Wg.f64, Wu.f64, bg.f64, bu.f64, 1, 0, ERF))
    print("  Y_0 %.2e" % e)
    assert e <= TOL["bf16"]


def test_gated_mlp_shards_reduce_to_the_unsharded_block():
    # every rank's gated share, its row-parallel partial, the on-device sum:
    # the oracle's unsharded gated block a(X Wg + bg) * (X Wu + bu) . W2
    w = inputs.Workload(53, "gated_mlp", "bf16", M=40, H=512, F=2048, T=4)
    X, Wg, Wu, bg, bu = inputs.gated_inputs(w)
    _, _, _, W2 = inputs.mlp_inputs(w)
    dW2t = W2.transposed().torch()
    parts = []
    for i in range(w.T):
        Y = run_gated(X, Wg, Wu, bg, bu, w.M, w.H, w.F, w.T, i, ERF, "bf16")
        Z = torch.empty(w.M, w.H, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(Y, dW2t, Z, w.M, w.H, w.F, w.T, i, tp.TP_BF16)
        parts.append(Z)
    out = torch.empty(w.M, w.H, dtype=torch.float32, device="cuda")
    tp.tp_shard_reduce(parts, w.T, None, out, None, w.M, w.H)
    torch.cuda.synchronize()
    Yfull = oracle.colpar_gated(X.f64, Wg.f64, Wu.f64, bg.f64, bu.f64, 1, 0, ERF)
    want = oracle.rowpar_partial(Yfull, W2.f64, 1, 0)
    e = rel_fro(to_f64(out), want)
    print("  Z %.2e" % e)
    assert e <= TOL["bf16"]
    assert np.isfinite(to_f64(out)).all()


# --------------------------------------- narrow grids (fewer blocks than CUs)
@pytest.mark.parametrize("M", [8, 32])
@pytest.mark.parametrize("kind", ["gelu", "gated", "rowpar"])
def test_narrow_skinny_grid(kind, M):
    # K = 4096 and fewer blocks than CUs: with one token tile (M = 8) the
    # skinny-M stream runs sixteen waves per block, with two (M = 32) eight
    # waves that regroup the token rows through LDS; every epilogue on both
    H = 4096
    if kind == "rowpar":
        # Z [8, 1024] = Y [8, 4096] . W2 [4096, 1024]: 64 blocks, K = 4096
        w = inputs.Workload(54, "narrow_rowpar", "bf16", M=M, H=1024, F=4096, T=1)
        _, _, _, W2 = inputs.mlp_inputs(w, M=M)
        Y = inputs.normal((M, 4096), 1.0, "bf16", seed=1, workload=54, tensor=inputs.X_ID)
        Z = torch.empty(M, 1024, dtype=torch.float32, device="cuda")
        tp.tp_rowpar_partial(Y.torch(), W2.transposed().torch(), Z, M, 1024, 4096, 1, 0, tp.TP_BF16)
        torch.cuda.synchronize()
        e = rel_fro(to_f64(Z), oracle.rowpar_partial(Y.f64, W2.f64, 1, 0))
    elif kind == "gelu":
        w = inputs.Workload(55, "narrow_gelu", "bf16", M=M, H=H, F=2048, T=2)
        X, W1, b1, _ = inputs.mlp_inputs(w, M=M)
        Y = torch.empty(M, 1024, dtype=torch.bfloat16, device="cuda")
        tp.tp_colpar_act(X.torch(), W1.transposed().torch(), b1.torch(), Y, M, H, 2048, 2, 1, tp.TP_GELU_ERF)
        torch.cuda.synchronize()
        e = rel_fro(to_f64(Y), oracle.colpar_act(X.f64, W1.f64, b1.f64, 2, 1, ERF))
    else:
        w = inputs.Workload(56, "narrow_gated", "bf16", M=M, H=H, F=2048, T=2)
        X, Wg, Wu, bg, bu = inputs.gated_inputs(w, M=M)
        Y = run_gated(X, Wg, Wu, bg, bu, M, H, 2048, 2, 0, TANH, "bf16")
        torch.cuda.synchronize()
        e = rel_fro(to_f64(Y), oracle.colpar_gated(X.f64, Wg.f64, Wu.f64, bg.f64, bu.f64, 2, 0, TANH))
    print("  %s %.2e" % (kind, e))
    assert e <= TOL["bf16"]
