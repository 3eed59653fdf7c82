"""The full 80-layer stack at its configured size, teacher-forced against the
fp64 oracle: H=8192, F=32768, A=64 heads x 128 = 8192, T=8, every rank of
the group emulated per layer, at decode M=8 and prefill M=4096.

"Tensor parallelism" (inference guide), "Walking through a transformer
block" and its 80-layer worked example fix the stack: per layer the
head-sharded attention out-projection and the MLP, each followed by an
all-reduce on the residual path ("Slice the matrix itself", "All-Reduce
Synchronization").  The layers checked here (0, 1, 40, 79) draw their
weights and attention context from the seeded host generator; the other
layers are drawn on the device with the same distributions.  For a checked
layer l the oracle is fed the GPU's residual stream h_l on a sample of
token rows (teacher forcing: no step of a layer mixes rows) and must
reproduce, within the bf16 tolerance, the GPU's increment h_{l+1} - h_l and
its row-RMS bf16 copy x_l.  At M=4096 the sample holds the first and last
row of every 256-row tile row plus seeded interior rows, and the error is
also checked per 256-row block.  The layers run the group launches the
bench times (batch-8 256x256 MFMA tiles at M=4096, the weight-streaming
kernels at M=8)."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_transformer_colpar_amd import inputs
from tests.harness import TOL, rel_fro, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from megatron_tensor_transformer_colpar_amd import tp

CHECK = (0, 1, 40, 79)
MMAX = 4096


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    say("\n[case] %s" % request.node.name)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def host_layers():
    """Seeded host draws of the checked layers: W_o [A,H], W1 [H,F], b1 [F],
    W2 [F,H] (logical [in, out]) and the T ctx shards [MMAX, A/T]."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    w = inputs.WORKLOADS["stack80"]
    As = w.A // w.T
    jobs = {}
    for l in CHECK:
        kw = dict(workload=w.wid, layer=l)
        jobs[(l, "Wo")] = ((w.A, w.H), w.w_std, dict(tensor=inputs.WO_ID, **kw))
        jobs[(l, "W1")] = ((w.H, w.F), w.w_std, dict(tensor=inputs.W1_ID, **kw))
        jobs[(l, "b1")] = ((w.F,), w.b_std, dict(tensor=inputs.B1_ID, **kw))
        jobs[(l, "W2")] = ((w.F, w.H), w.w_std, dict(tensor=inputs.W2_ID, **kw))
        for i in range(w.T):
            jobs[(l, "ctx%d" % i)] = ((MMAX, As), 1.0, dict(tensor=inputs.CTX_ID, shard=i + 1, **kw))
    say("  drawing %d host tensors of layers %s" % (len(jobs), CHECK))
    with ThreadPoolExecutor(max_workers=8) as ex:
        futs = {k: ex.submit(inputs.normal, shape, std, "bf16", **kw) for k, (shape, std, kw) in jobs.items()}
        out = {k: f.result() for k, f in futs.items()}
    say("  host draws done")
    return {l: dict(Wo=out[(l, "Wo")], W1=out[(l, "W1")], b1=out[(l, "b1")], W2=out[(l, "W2")],
                    ctx=[out[(l, "ctx%d" % i)] for i in range(w.T)]) for l in CHECK}


def stored(t):
    """Upload a logical [in, out] bf16 weight and store it K-contiguous
    ([out, in]); the transpose is device-side data movement only."""
    return t.torch().t().contiguous()


@pytest.fixture(scope="module")
def device_layers(host_layers):
    w = inputs.WORKLOADS["stack80"]
    H, F, A = w.H, w.F, w.A
    g = torch.Generator(device="cuda").manual_seed(17)
    layers = []
    for l in range(w.layers):
        if l in host_layers:
            hl = host_layers[l]
            layers.append(dict(Wot=stored(hl["Wo"]), W1t=stored(hl["W1"]), b1=hl["b1"].torch(), W2t=stored(hl["W2"])))
        else:
            layers.append(dict(Wot=(torch.randn(H, A, generator=g, device="cuda") * w.w_std).to(torch.bfloat16),
                               W1t=(torch.randn(F, H, generator=g, device="cuda") * w.w_std).to(torch.bfloat16),
                               b1=(torch.randn(F, generator=g, device="cuda") * w.b_std).to(torch.bfloat16),
                               W2t=(torch.randn(H, F, generator=g, device="cuda") * w.w_std).to(torch.bfloat16)))
    torch.cuda.synchronize()
    say("  %d layers on the device" % len(layers))
    yield layers, g
    del layers
    torch.cuda.empty_cache()


def tile_row_sample(M, extra, seed):
    """First and last row of every 256-row tile row, plus `extra` seeded rows."""
    ends = {r for t in range(0, M, 256) for r in (t, min(M, t + 256) - 1)}
    return np.array(sorted(ends | set(inputs.row_sample(M, extra, seed=seed).tolist())), dtype=np.int64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("M", [8, 4096])
def test_stack80_teacher_forced(M, host_layers, device_layers):
    w = inputs.WORKLOADS["stack80"]
    H, F, A, T = w.H, w.F, w.A, w.T
    layers, g = device_layers
    rows = np.arange(M) if M <= 32 else tile_row_sample(M, 32, seed=M)
    rows_t = torch.from_numpy(rows).cuda()
    # ctx: host draws (first M rows) for the checked layers, device draws elsewhere
    ctx_t = []
    for l in range(w.layers):
        if l in host_layers:
            ctx_t.append([c.rows(slice(0, M)).torch() for c in host_layers[l]["ctx"]])
        else:
            ctx_t.append([torch.randn(M, A // T, generator=g, device="cuda").to(torch.bfloat16) for _ in range(T)])
    ctx = [tp.partial_array(c) for c in ctx_t]
    X = inputs.normal((M, H), w.x_std, "bf16", workload=w.wid, tensor=inputs.X_ID)
    h = X.torch().float()
    xhat = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    Y_t = [torch.empty(M, F // T, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
    P_t = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]
    Y, parts = tp.partial_array(Y_t), tp.partial_array(P_t)
    snaps = {}
    for l, p in enumerate(layers):
        h_in = h.index_select(0, rows_t).clone() if l in host_layers else None
        tp.tp_layer_fwd(h, xhat, ctx[l], p["Wot"], A, p["W1t"], p["b1"], p["W2t"], Y, parts, M, H, F, T)
        if l in host_layers:
            snaps[l] = (h_in, h.index_select(0, rows_t).clone(), xhat.index_select(0, rows_t).clone())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(h).all())
    say("  stack done; rows checked: %d of %d" % (len(rows), M))
    worst = 0.0
    for l in CHECK:
        hl = host_layers[l]
        h_in, h_out, xh = (to_f64(t) for t in snaps[l])
        if l == 0:   # layer 0's input is the host draw itself
            assert np.array_equal(h_in, X.f64[rows])
        ctx_rows = [c.f64[rows] for c in hl["ctx"]]
        ref_out, ref_xh = oracle.layer_fwd(h_in, ctx_rows, hl["Wo"].f64, hl["W1"].f64, hl["b1"].f64, hl["W2"].f64, T,
                                           tp.TP_RMS_EPS)
        e_inc = rel_fro(h_out - h_in, ref_out - h_in)
        e_h, e_x = rel_fro(h_out, ref_out), rel_fro(xh, ref_xh)
        say("  layer %2d: increment %.2e  h %.2e  xhat %.2e  (rms h_in %.1f)"
            % (l, e_inc, e_h, e_x, float(np.sqrt(np.mean(h_in ** 2)))))
        assert e_inc <= TOL["bf16"] and e_h <= TOL["bf16"] and e_x <= TOL["bf16"], l
        worst = max(worst, e_inc, e_x)
        if M > 32:   # per 256-row block of the sample
            blocks = rows // 256
            for b in np.unique(blocks):
                sel = blocks == b
                eb = rel_fro((h_out - h_in)[sel], (ref_out - h_in)[sel])
                assert eb <= TOL["bf16"], (l, int(b), eb)
    say("  worst over checked layers: %.2e" % worst)
