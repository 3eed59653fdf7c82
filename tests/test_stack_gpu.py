"""The layer stack (per layer: head-sharded out-projection of all ranks, the
reduce into the residual stream with its row-RMS bf16 copy, all ranks' MLP
shares, the second reduce) against the fp64 oracle, free-running from the
same seeded inputs; and properties of the full 80-layer stack that hold at
any size."""
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


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def host_layer(w, layer, M, T, A):
    """Seeded inputs of one layer: ctx shards, W_o [A,H], W1 [H,F], b1, W2 [F,H]."""
    kw = dict(workload=w.wid, layer=layer)
    ctx = [inputs.normal((M, A // T), 1.0, "bf16", tensor=inputs.CTX_ID, shard=i + 1, **kw) for i in range(T)]
    Wo = inputs.normal((A, w.H), w.w_std, "bf16", tensor=inputs.WO_ID, **kw)
    W1 = inputs.normal((w.H, w.F), w.w_std, "bf16", tensor=inputs.W1_ID, **kw)
    b1 = inputs.normal((w.F,), w.b_std, "bf16", tensor=inputs.B1_ID, **kw)
    W2 = inputs.normal((w.F, w.H), w.w_std, "bf16", tensor=inputs.W2_ID, **kw)
    return ctx, Wo, W1, b1, W2


class DeviceStack:
    def __init__(self, M, H, F, A, T):
        self.M, self.H, self.F, self.A, self.T = M, H, F, A, T
        self.xhat = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
        self.Y = [torch.empty(M, F // T, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
        self.parts = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]

    def layer(self, h, ctx, Wot, W1t, b1, W2t):
        tp.tp_layer_fwd(h, self.xhat, ctx, Wot, self.A, W1t, b1, W2t, self.Y, self.parts,
                        self.M, self.H, self.F, self.T)


@pytest.mark.parametrize("M", [8, 40])
def test_small_stack_free_running(M):
    w = inputs.Workload(30, "stack_small", "bf16", M=M, H=512, F=2048, T=8, A=512, layers=4)
    X = inputs.normal((M, w.H), 1.0, "bf16", workload=w.wid, tensor=inputs.X_ID)
    st = DeviceStack(M, w.H, w.F, w.A, w.T)
    h = X.torch().float()
    href = X.f64
    for l in range(w.layers):
        ctx, Wo, W1, b1, W2 = host_layer(w, l, M, w.T, w.A)
        st.layer(h, [c.torch() for c in ctx], Wo.transposed().torch(), W1.transposed().torch(), b1.torch(),
                 W2.transposed().torch())
        torch.cuda.synchronize()
        href, xref = oracle.layer_fwd(href, [c.f64 for c in ctx], Wo.f64, W1.f64, b1.f64, W2.f64, w.T,
                                      tp.TP_RMS_EPS)
        eh, ex = rel_fro(to_f64(h), href), rel_fro(to_f64(st.xhat), xref)
        print("  layer %d: h %.2e  xhat %.2e" % (l, eh, ex))
        assert eh <= TOL["bf16"] and ex <= TOL["bf16"]


def test_full_width_layer():
    # H=8192, F=32768, A=64 heads x 128, T=8, M=8: one layer of the stack
    w = inputs.WORKLOADS["stack80"]
    M = w.M
    X = inputs.normal((M, w.H), 1.0, "bf16", workload=w.wid, tensor=inputs.X_ID)
    ctx, Wo, W1, b1, W2 = host_layer(w, 0, M, w.T, w.A)
    st = DeviceStack(M, w.H, w.F, w.A, w.T)
    h = X.torch().float()
    st.layer(h, [c.torch() for c in ctx], Wo.transposed().torch(), W1.transposed().torch(), b1.torch(),
             W2.transposed().torch())
    torch.cuda.synchronize()
    href, xref = oracle.layer_fwd(X.f64, [c.f64 for c in ctx], Wo.f64, W1.f64, b1.f64, W2.f64, w.T, tp.TP_RMS_EPS)
    eh, ex = rel_fro(to_f64(h), href), rel_fro(to_f64(st.xhat), xref)
    print("  h %.2e  xhat %.2e" % (eh, ex))
    assert eh <= TOL["bf16"] and ex <= TOL["bf16"]


def device_layers(L, H, F, A, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for _ in range(L):
        out.append(dict(Wot=(torch.randn(H, A, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
                        W1t=(torch.randn(F, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
                        b1=(torch.randn(F, generator=g, device="cuda") * 0.01).to(torch.bfloat16),
                        W2t=(torch.randn(H, F, generator=g, device="cuda") * 0.02).to(torch.bfloat16)))
    return out, g


def test_stack80_properties():
    # the full 80-layer stack at H=8192, F=32768, T=8, M=8: finite, xhat has
    # unit row RMS at every layer, the residual stream grows, and two runs
    # agree bit for bit
    w = inputs.WORKLOADS["stack80"]
    M, H, F, A, T = w.M, w.H, w.F, w.A, w.T
    layers, g = device_layers(w.layers, H, F, A, seed=5)
    ctxs = [[torch.randn(M, A // T, generator=g, device="cuda").to(torch.bfloat16) for _ in range(T)]
            for _ in range(w.layers)]
    x0 = torch.randn(M, H, generator=g, device="cuda").to(torch.bfloat16).float()
    st = DeviceStack(M, H, F, A, T)
    runs = []
    for rep in range(2):
        h = x0.clone()
        rms = []
        for l, p in enumerate(layers):
            st.layer(h, ctxs[l], p["Wot"], p["W1t"], p["b1"], p["W2t"])
            if rep == 0 and l % 16 == 0:
                rms.append(st.xhat.float().pow(2).mean(dim=1).sqrt())
        torch.cuda.synchronize()
        runs.append(h)
        if rep == 0:
            for r in rms:
                assert torch.allclose(r, torch.ones_like(r), atol=1e-2)
    assert bool(torch.isfinite(runs[0]).all())
    assert torch.equal(runs[0], runs[1])
    assert float(runs[0].pow(2).mean()) > float(x0.pow(2).mean())
