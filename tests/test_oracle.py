"""Pins for the fp64 oracle, checked against what the pages and mathematics fix.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign or constant, a transposed operand, a wrong shard offset, a missing
bias) fails at least one of them; ``test_oracle_mutants.py`` plants such
mistakes in a copy of the oracle and checks that they are caught.

Sources: "Slice the matrix itself" (column/row-parallel GEMMs, row-parallel
summation); "09. Tensor Parallelism in Action" section 1 (block split) and
section 2 question 2 (GeLU commutes with the column split); "Tensor
parallelism" guide, "Concept".  GeLU: Hendrycks & Gimpel, arXiv:1606.08415.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _phi_gelu(x):
    """Exact GELU x * Phi(x) through the C library's erf."""
    return np.array([v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0))) for v in np.ravel(x)])


# ---------------------------------------------------------------- GeLU pins
def test_gelu_odd_part_identity():
    # tanh is odd, so g(x) - g(-x) = x exactly in real arithmetic.
    x = np.linspace(-10, 10, 40001)
    d = oracle.gelu(x) - oracle.gelu(-x)
    assert np.max(np.abs(d - x) / (1 + np.abs(x))) < 4e-15


def test_gelu_tanh_form_error_against_exact_gelu():
    # The tanh form approximates x*Phi(x); its largest deviation on the real
    # line is 4.73e-4 near |x| = 2.70.  A dropped cubic term (3.4e-2), a wrong
    # scale sqrt(pi/2) (9.2e-2), x^2 for x^3 (5.9e-2) or a mistyped 0.04715
    # (1.5e-3) all land far outside this band.
    x = np.linspace(-10, 10, 200001)
    err = np.abs(oracle.gelu(x) - _phi_gelu(x))
    assert 4.70e-4 < err.max() < 4.76e-4
    assert abs(abs(x[err.argmax()]) - 2.70) < 0.01


def test_gelu_special_values():
    g = oracle.gelu(np.array([0.0, 30.0, -30.0, 1e-8, -1e-8]))
    assert g[0] == 0.0
    assert g[1] == 30.0            # g(x) -> x for large x
    assert abs(g[2]) < 1e-300      # g(x) -> 0 for large negative x
    # slope 1/2 at the origin: g(x) = x/2 + O(x^2)
    assert abs(g[3] / 1e-8 - 0.5) < 1e-7 and abs(g[4] / -1e-8 - 0.5) < 1e-7


def test_gelu_high_precision_values():
    # Rounding check of the fp64 evaluation against 40-digit arithmetic.
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 40
    xs = [-3.0, -1.0, -0.5, 0.5, 1.0, 2.0, 3.0, 7.25]
    k = mp.sqrt(2 / mp.pi)
    ref = [float(mp.mpf(0.5) * x * (1 + mp.tanh(k * (x + mp.mpf("0.044715") * x ** 3)))) for x in xs]
    got = oracle.gelu(np.array(xs))
    # 1 + tanh(.) cancels for negative x, so the bound scales with |x|.
    for x, r, g in zip(xs, ref, got):
        assert abs(g - r) <= 8 * np.finfo(np.float64).eps * (1 + abs(x))


# -------------------------------------- exact GeLU (x * Phi(x), erf form)
ERF, TANH = oracle.ACT_GELU_ERF, oracle.ACT_GELU_TANH


def test_gelu_erf_textbook_values():
    # g(x) = x * Phi(x): Phi(1) = 0.8413447460685429 and the two-sided 95%
    # normal quantile Phi(1.959963984540054) = 0.975 are table values.
    g1 = oracle.act(np.array([1.0, -1.0]), ERF)
    assert abs(g1[0] - 0.8413447460685429) < 2e-16
    assert abs(g1[1] - (-(1.0 - 0.8413447460685429))) < 2e-16
    q = 1.959963984540054
    assert abs(oracle.act(np.array([q]), ERF)[0] / q - 0.975) < 1e-15


def test_gelu_erf_odd_part_identity_and_limits():
    # Phi(x) + Phi(-x) = 1, so g(x) - g(-x) = x.
    x = np.linspace(-10, 10, 40001)
    d = oracle.act(x, ERF) - oracle.act(-x, ERF)
    assert np.max(np.abs(d - x) / (1 + np.abs(x))) < 4e-15
    g = oracle.act(np.array([0.0, 40.0, -40.0, 1e-8]), ERF)
    assert g[0] == 0.0 and g[1] == 40.0 and abs(g[2]) < 1e-300
    assert abs(g[3] / 1e-8 - 0.5) < 1e-7


def test_gelu_erf_high_precision_values():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 40
    xs = [-6.0, -3.0, -1.0, -0.5, -1e-3, 1e-3, 0.5, 2.0, 3.0, 7.25]
    ref = [float(mp.mpf(x) * (1 + mp.erf(mp.mpf(x) / mp.sqrt(2))) / 2) for x in xs]
    got = oracle.act(np.array(xs), ERF)
    for x, r, g in zip(xs, ref, got):
        assert abs(g - r) <= 8 * np.finfo(np.float64).eps * (1 + abs(x))


def test_gelu_forms_differ_by_the_published_bound():
    # The tanh form's largest deviation from x*Phi(x) is 4.73e-4 at |x| ~ 2.70,
    # and the tanh entry points agree with each other bit for bit.
    x = np.linspace(-10, 10, 200001)
    t, e = oracle.act(x, TANH), oracle.act(x, ERF)
    assert np.array_equal(t, oracle.gelu(x))
    err = np.abs(t - e)
    assert 4.70e-4 < err.max() < 4.76e-4
    assert abs(abs(x[err.argmax()]) - 2.70) < 0.01


# ------------------------------------------------------ column-parallel pins
def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_colpar_gelu_matches_library_matmul():
    rng = np.random.default_rng(1)
    M, H, F, T = 7, 48, 40, 4
    X, W1, b1 = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F)
    for i in range(T):
        C = slice(i * F // T, (i + 1) * F // T)
        want = oracle.gelu(X @ W1[:, C] + b1[C])
        got = oracle.colpar_gelu(X, W1, b1, T, i)
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want)))


def test_colpar_gelu_bruteforce_integers():
    # Small integers: every partial sum is exact in fp64, so the pre-activation
    # is known exactly from Python integer arithmetic, whatever the order.
    rng = np.random.default_rng(2)
    M, H, F, T = 3, 5, 6, 3
    X = rng.integers(-4, 5, (M, H))
    W1 = rng.integers(-4, 5, (H, F))
    b1 = rng.integers(-4, 5, F)
    for i in range(T):
        Fs = F // T
        pre = [[sum(int(X[m, h]) * int(W1[h, i * Fs + c]) for h in range(H)) + int(b1[i * Fs + c])
                for c in range(Fs)] for m in range(M)]
        want = oracle.gelu(np.array(pre, dtype=np.float64))
        assert np.array_equal(oracle.colpar_gelu(X, W1, b1, T, i), want)


def test_colpar_gelu_closed_forms():
    rng = np.random.default_rng(3)
    M, H, F, T = 4, 8, 12, 3
    c = _rand(rng, F)
    # W1 = 0: every row is g(b1[C_i])
    Y = oracle.colpar_gelu(_rand(rng, M, H), np.zeros((H, F)), c, T, 1)
    assert np.array_equal(Y, np.tile(oracle.gelu(c[4:8]), (M, 1)))
    # X = e_k: row picks out W1[k, C_i] + b1[C_i]
    W1 = _rand(rng, H, F)
    X = np.zeros((1, H))
    X[0, 5] = 1.0
    Y = oracle.colpar_gelu(X, W1, c, T, 2)
    assert np.array_equal(Y[0], oracle.gelu(W1[5, 8:12] + c[8:12]))
    # no bias equals zero bias
    Xr = _rand(rng, M, H)
    assert np.array_equal(oracle.colpar_gelu(Xr, W1, None, T, 0),
                          oracle.colpar_gelu(Xr, W1, np.zeros(F), T, 0))


def test_colpar_act_erf_matches_library_matmul_and_closed_forms():
    rng = np.random.default_rng(30)
    M, H, F, T = 5, 16, 12, 3
    X, W1, b1 = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F)
    for i in range(T):
        C = slice(i * F // T, (i + 1) * F // T)
        want = oracle.act(X @ W1[:, C] + b1[C], ERF)
        got = oracle.colpar_act(X, W1, b1, T, i, ERF)
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want)))
    # W1 = 0: every row is g(b1[C_i]); the tanh form is colpar_gelu
    Y = oracle.colpar_act(X, np.zeros((H, F)), b1, T, 2, ERF)
    assert np.array_equal(Y, np.tile(oracle.act(b1[8:12], ERF), (M, 1)))
    assert np.array_equal(oracle.colpar_act(X, W1, b1, T, 1, TANH), oracle.colpar_gelu(X, W1, b1, T, 1))


# ------------------------------------------------- gated first layer pins
def test_gated_hand_example():
    # H = 1, F = 2, T = 2: X = [1; 2], Wg = [1, -1], Wu = [3, 2], no biases.
    # Rank 0 owns column 0: g(x) * 3x; rank 1 owns column 1: g(-x) * 2x.
    X, Wg, Wu = np.array([[1.0], [2.0]]), np.array([[1.0, -1.0]]), np.array([[3.0, 2.0]])
    phi1 = 0.8413447460685429
    y0 = oracle.colpar_gated(X, Wg, Wu, None, None, 2, 0, ERF)
    y1 = oracle.colpar_gated(X, Wg, Wu, None, None, 2, 1, ERF)
    assert abs(y0[0, 0] - phi1 * 3.0) < 1e-15
    assert abs(y1[0, 0] - (-(1.0 - phi1)) * 2.0) < 1e-15
    assert abs(y0[1, 0] - oracle.act(np.array([2.0]), ERF)[0] * 6.0) < 1e-15


def test_gated_reduces_to_plain_forms():
    rng = np.random.default_rng(31)
    M, H, F, T = 6, 10, 8, 2
    X, Wg, Wu, bg, bu = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, H, F), _rand(rng, F), _rand(rng, F)
    for form in (TANH, ERF):
        for i in range(T):
            C = slice(i * F // T, (i + 1) * F // T)
            # gate weights 0, gate bias c: a(c) scales the up projection
            got = oracle.colpar_gated(X, np.zeros((H, F)), Wu, bg, bu, T, i, form)
            want = oracle.act(bg[C], form) * (X @ Wu[:, C] + bu[C])
            assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want)))
            # up weights 0, up bias 1: the plain column-parallel activation
            got = oracle.colpar_gated(X, Wg, np.zeros((H, F)), bg, np.ones(F), T, i, form)
            assert np.array_equal(got, oracle.colpar_act(X, Wg, bg, T, i, form))
    # gate and up are not interchangeable
    a = oracle.colpar_gated(X, Wg, Wu, bg, bu, T, 0, ERF)
    b = oracle.colpar_gated(X, Wu, Wg, bu, bg, T, 0, ERF)
    assert np.max(np.abs(a - b)) > 0.1


def test_gated_bruteforce_integers():
    rng = np.random.default_rng(32)
    M, H, F, T = 3, 5, 6, 3
    X, Wg, Wu = (rng.integers(-3, 4, s) for s in ((M, H), (H, F), (H, F)))
    bg, bu = rng.integers(-3, 4, F), rng.integers(-3, 4, F)
    Fs = F // T
    for form in (TANH, ERF):
        for i in range(T):
            pg = np.array([[sum(int(X[m, h]) * int(Wg[h, i * Fs + c]) for h in range(H)) + int(bg[i * Fs + c])
                            for c in range(Fs)] for m in range(M)], dtype=np.float64)
            pu = np.array([[sum(int(X[m, h]) * int(Wu[h, i * Fs + c]) for h in range(H)) + int(bu[i * Fs + c])
                            for c in range(Fs)] for m in range(M)], dtype=np.float64)
            assert np.array_equal(oracle.colpar_gated(X, Wg, Wu, bg, bu, T, i, form), oracle.act(pg, form) * pu)


def test_gated_shards_concatenate_to_unsharded():
    rng = np.random.default_rng(33)
    M, H, F = 4, 12, 16
    X, Wg, Wu, bg, bu = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, H, F), _rand(rng, F), None
    full = oracle.colpar_gated(X, Wg, Wu, bg, bu, 1, 0, ERF)
    for T in (2, 4, 8):
        cat = np.concatenate([oracle.colpar_gated(X, Wg, Wu, bg, bu, T, i, ERF) for i in range(T)], axis=1)
        assert np.array_equal(cat, full)


# --------------------------------------------------------- row-parallel pins
def test_rowpar_partial_bruteforce_integers():
    rng = np.random.default_rng(4)
    M, H, F, T = 3, 4, 8, 2
    Yi = rng.integers(-5, 6, (M, F // T))
    W2 = rng.integers(-5, 6, (F, H))
    for i in range(T):
        want = [[sum(int(Yi[m, c]) * int(W2[i * F // T + c, n]) for c in range(F // T))
                 for n in range(H)] for m in range(M)]
        assert np.array_equal(oracle.rowpar_partial(Yi, W2, T, i), np.array(want, dtype=np.float64))


def test_rowpar_partial_matches_library_matmul_and_is_linear():
    rng = np.random.default_rng(5)
    M, H, F, T = 6, 20, 32, 4
    W2 = _rand(rng, F, H)
    for i in range(T):
        Yi = _rand(rng, M, F // T)
        want = Yi @ W2[i * F // T:(i + 1) * F // T]
        got = oracle.rowpar_partial(Yi, W2, T, i)
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want)))
        # scaling by a power of two is exact
        assert np.array_equal(oracle.rowpar_partial(Yi, 4.0 * W2, T, i), 4.0 * got)


# ------------------------------------------------------- split-algebra pins
@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_shard_sum_equals_unsharded(T):
    # Row-parallel partials sum to the unsharded product, and the concatenated
    # column shards are the unsharded activation bit for bit (GeLU is
    # elementwise, so it commutes with the column split).
    rng = np.random.default_rng(10 + T)
    M, H, F = 5, 24, 64
    X, W1, b1, W2 = _rand(rng, M, H), 0.2 * _rand(rng, H, F), 0.1 * _rand(rng, F), 0.2 * _rand(rng, F, H)
    Y, Z = oracle.mlp_unsharded(X, W1, b1, W2)
    parts = [oracle.mlp_shard(X, W1, b1, W2, T, i) for i in range(T)]
    assert np.array_equal(np.concatenate([p[0] for p in parts], axis=1), Y)
    Zsum = oracle.shard_reduce(np.stack([p[1] for p in parts]))
    assert np.linalg.norm(Zsum - Z) <= 1e-13 * np.linalg.norm(Z)


@settings(max_examples=40, deadline=None)
@given(M=st.integers(1, 9), H=st.integers(1, 17), Fs=st.integers(1, 6),
       T=st.sampled_from([1, 2, 3, 4, 8]), seed=st.integers(0, 2**31 - 1))
def test_shard_sum_equals_unsharded_any_shape(M, H, Fs, T, seed):
    rng = np.random.default_rng(seed)
    F = Fs * T
    X, W1, b1, W2 = _rand(rng, M, H), _rand(rng, H, F), _rand(rng, F), _rand(rng, F, H)
    Y, Z = oracle.mlp_unsharded(X, W1, b1, W2)
    Ys, Zs = zip(*[oracle.mlp_shard(X, W1, b1, W2, T, i) for i in range(T)])
    assert np.array_equal(np.concatenate(Ys, axis=1), Y)
    assert np.linalg.norm(sum(Zs) - Z) <= 1e-12 * (1 + np.linalg.norm(Z))
    # the unsharded block against the library matmul
    Z_lib = oracle.gelu(X @ W1 + b1) @ W2
    assert np.linalg.norm(Z - Z_lib) <= 1e-12 * (1 + np.linalg.norm(Z_lib))


def test_hand_example_two_ranks():
    # X = [1, 2], W1 = W2 = I, no bias, T = 2: rank 0 owns column 0 and rank 1
    # column 1, so the partials are [g(1), 0] and [0, g(2)].
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 30
    k = mp.sqrt(2 / mp.pi)
    g = lambda x: float(mp.mpf(0.5) * x * (1 + mp.tanh(k * (x + mp.mpf("0.044715") * x ** 3))))
    X, I = np.array([[1.0, 2.0]]), np.eye(2)
    _, Z0 = oracle.mlp_shard(X, I, None, I, 2, 0)
    _, Z1 = oracle.mlp_shard(X, I, None, I, 2, 1)
    assert abs(Z0[0, 0] - g(1)) < 1e-15 and Z0[0, 1] == 0.0
    assert Z1[0, 0] == 0.0 and abs(Z1[0, 1] - g(2)) < 1e-15
    assert abs(g(1) - 0.8411919906082767) < 1e-15 and abs(g(2) - 1.954597694087775) < 1e-15


# ------------------------------------------------------------- reduce pins
def test_reduce_integers_exact_with_residual():
    rng = np.random.default_rng(6)
    T, M, H = 8, 3, 10
    P = rng.integers(-1000, 1000, (T, M, H)).astype(np.float64)
    R = rng.integers(-1000, 1000, (M, H)).astype(np.float64)
    want = np.array([[int(R[m, n]) + sum(int(P[j, m, n]) for j in range(T)) for n in range(H)]
                     for m in range(M)], dtype=np.float64)
    assert np.array_equal(oracle.shard_reduce(P, R), want)
    assert np.array_equal(oracle.shard_reduce(P[:1]), P[0])


def test_reduce_rms_closed_forms():
    # constant row c: c / sqrt(c^2 + eps);  row [3, 4]: mean square 12.5
    P = np.zeros((2, 2, 2))
    P[0] = [[1.5, 1.5], [3.0, 4.0]]
    P[1] = [[1.5, 1.5], [0.0, 0.0]]
    out, rms = oracle.shard_reduce(P, rms_eps=1e-6)
    assert np.array_equal(out, [[3.0, 3.0], [3.0, 4.0]])
    assert np.allclose(rms[0], 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15, atol=0)
    assert np.allclose(rms[1], np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6), rtol=1e-15, atol=0)
    # unit RMS after normalisation (eps negligible)
    rng = np.random.default_rng(7)
    _, r = oracle.shard_reduce(rng.standard_normal((3, 4, 64)) * 5, rms_eps=1e-12)
    assert np.allclose(np.sqrt(np.mean(r ** 2, axis=1)), 1.0, rtol=1e-12)


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.act(np.ones(3), 7)                                         # unknown form
    with pytest.raises(ValueError):
        oracle.colpar_gated(np.ones((2, 3)), np.ones((3, 4)), np.ones((3, 5)), None, None, 2, 0, ERF)
    with pytest.raises(ValueError):
        oracle.colpar_gelu(np.ones((2, 3)), np.ones((3, 5)), None, 2, 0)   # F % T
    with pytest.raises(ValueError):
        oracle.colpar_gelu(np.ones((2, 3)), np.ones((3, 4)), None, 2, 2)   # i >= T
    with pytest.raises(ValueError):
        oracle.rowpar_partial(np.ones((2, 3)), np.ones((4, 5)), 2, 0)      # Y_i width


# ------------------------------------------------------- layer-stack pins
def _layer_inputs(rng, M=3, H=16, F=32, A=16, T=4):
    ctx = [rng.standard_normal((M, A // T)) for _ in range(T)]
    return (rng.standard_normal((M, H)), ctx, 0.3 * rng.standard_normal((A, H)),
            0.3 * rng.standard_normal((H, F)), 0.1 * rng.standard_normal(F), 0.3 * rng.standard_normal((F, H)))


def test_layer_zero_weights_leave_the_stream_unchanged():
    rng = np.random.default_rng(20)
    h, ctx, Wo, W1, b1, W2 = _layer_inputs(rng)
    out, xh = oracle.layer_fwd(h, ctx, 0 * Wo, W1, b1, 0 * W2, 4, 1e-6)
    assert np.array_equal(out, h)
    assert np.allclose(np.sqrt(np.mean(xh ** 2, axis=1)), 1.0, rtol=1e-6)


def test_layer_is_independent_of_the_tp_degree():
    # Sharding does not change the mathematics: T = 1, 2, 4 give the same block.
    rng = np.random.default_rng(21)
    h, _, Wo, W1, b1, W2 = _layer_inputs(rng)
    ctx_full = rng.standard_normal((3, 16))
    outs = []
    for T in (1, 2, 4):
        ctx = [ctx_full[:, i * 16 // T:(i + 1) * 16 // T] for i in range(T)]
        outs.append(oracle.layer_fwd(h, ctx, Wo, W1, b1, W2, T, 1e-6)[0])
    assert np.allclose(outs[0], outs[1], rtol=0, atol=1e-12) and np.allclose(outs[0], outs[2], rtol=0, atol=1e-12)


def test_layer_against_library_composition():
    # the same block from numpy's matmul and the pinned GeLU
    rng = np.random.default_rng(22)
    h, ctx, Wo, W1, b1, W2 = _layer_inputs(rng)
    out, _ = oracle.layer_fwd(h, ctx, Wo, W1, b1, W2, 4, 1e-6)
    h1 = h + np.concatenate(ctx, axis=1) @ Wo
    xh = h1 / np.sqrt(np.mean(h1 ** 2, axis=1, keepdims=True) + 1e-6)
    want = h1 + oracle.gelu(xh @ W1 + b1) @ W2
    assert np.max(np.abs(out - want)) <= 1e-12 * (1 + np.max(np.abs(want)))
