"""tp_mlp_shard_fwd_noalloc (Y_i staged in the library's own device buffer,
for callers that cannot allocate) against tp_mlp_shard_fwd (Y_i in a caller
workspace) through the C ABI: two calls in a row on the same GPU, the second
with a smaller input, each compared with the existing entry point (same
kernels, so bit for bit) and with the fp64 oracle on sampled rows."""
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


def one_call(w, M, T, i, rows):
    X, W1, b1, W2 = inputs.mlp_inputs(w, M=M)
    dev = DeviceMLP(X, W1, b1, W2)
    Fs = w.F // T
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    Z_ref = torch.empty(M, w.H, dtype=torch.float32, device="cuda")
    tp.tp_mlp_shard_fwd(dev.X, dev.W1t, dev.b1, dev.W2t, Y, Z_ref, M, w.H, w.F, T, i, tp.TP_BF16)
    Z = torch.full((M, w.H), float("nan"), dtype=torch.float32, device="cuda")
    tp.tp_mlp_shard_fwd_noalloc(dev.X, dev.W1t, dev.b1, dev.W2t, Z, M, w.H, w.F, T, i, tp.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z_ref)
    _, Zr = oracle.mlp_shard(X.f64[rows], W1.f64, b1.f64, W2.f64, T, i)
    e = rel_fro(to_f64(Z)[rows], Zr)
    print("  M=%d T=%d i=%d: bitwise equal to tp_mlp_shard_fwd; vs oracle %.2e" % (M, T, i, e))
    assert e <= TOL["bf16"]


def test_noalloc_two_calls_second_smaller():
    # first call at the staging limit: 2048 tokens x F/T = 4096 bf16 = 16 MiB
    # (MFMA GEMM path); the second a decode step of 8 tokens (weight-streaming
    # path) that reuses the start of the same buffer
    big = inputs.Workload(40, "noalloc_prefill", "bf16", M=2048, H=4096, F=16384, T=4)
    assert 2048 * (big.F // big.T) * 2 == tp.TP_NOALLOC_SCRATCH_BYTES
    one_call(big, 2048, big.T, 3, inputs.row_sample(2048, 24))
    small = inputs.Workload(41, "noalloc_decode", "bf16", M=8, H=8192, F=32768, T=8)
    one_call(small, 8, small.T, 5, np.arange(8))


def test_noalloc_over_the_limit_is_rejected_on_the_gpu_too():
    X = torch.zeros(2049, 64, dtype=torch.bfloat16, device="cuda")
    W1t = torch.zeros(4096, 64, dtype=torch.bfloat16, device="cuda")
    W2t = torch.zeros(64, 4096, dtype=torch.bfloat16, device="cuda")
    Z = torch.zeros(2049, 64, dtype=torch.float32, device="cuda")
    st = tp.raw.tp_mlp_shard_fwd_noalloc(X.data_ptr(), W1t.data_ptr(), None, W2t.data_ptr(), Z.data_ptr(),
                                         2049, 64, 4096, 1, 0, tp.TP_BF16, None)
    assert st == tp.TP_ERR_UNSUPPORTED and "limit" in tp.last_error()
