"""Pins of the oracle's backward pass of a rank's MLP share and of the GeLU
derivative, independent of their formulas: finite differences of the
oracle's own forward (itself pinned in test_oracle.py), textbook values,
closed-form identities, exact integer products, and the shard algebra (the
ranks' dX partials sum to the unsharded dX; the ranks' weight-gradient
blocks are the unsharded gradient's blocks).

Sources: "Slice the matrix itself", "Strict NVLink Domain Constraint"
(all-reduces on every layer, forward and backward); the "Megatron Internals
II" summary on the Tensor Parallel tag page (each parallel layer's contract
names the gradient path that communicates); Hendrycks & Gimpel, arXiv:1606.08415 (GeLU and its exact form).
Everything runs on the CPU.
"""
import math

import numpy as np
import pytest

import oracle

TANH, ERF, NONE = oracle.ACT_GELU_TANH, oracle.ACT_GELU_ERF, oracle.ACT_NONE


def _rng(seed):
    return np.random.default_rng(seed)


def test_gelu_grad_textbook_values():
    # exact form: g'(x) = Phi(x) + x phi(x); Phi(1) = 0.841344746..., phi(1) = 0.241970724...
    g = oracle.act_grad(np.array([0.0, 1.0, -1.0]), ERF)
    assert g[0] == 0.5
    assert abs(g[1] - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    assert abs(g[2] - (0.15865525393145707 - 0.24197072451914337)) < 1e-15
    assert oracle.act_grad(np.array([0.0]), TANH)[0] == 0.5
    x = _rng(1).standard_normal(16)
    assert np.array_equal(oracle.act_grad(x, NONE), np.ones(16))


@pytest.mark.parametrize("form", [TANH, ERF])
def test_gelu_grad_is_the_derivative_of_gelu(form):
    # central differences of the (pinned) forward g
    x = np.linspace(-6.0, 6.0, 241)
    h = 1e-5
    fd = (oracle.act(x + h, form) - oracle.act(x - h, form)) / (2 * h)
    assert np.max(np.abs(fd - oracle.act_grad(x, form))) < 1e-9


@pytest.mark.parametrize("form", [TANH, ERF])
def test_gelu_grad_odd_part_identity(form):
    # g(x) - g(-x) = x for both forms, so g'(x) + g'(-x) = 1; limits 0 and 1
    x = np.concatenate([np.linspace(-8, 8, 161), _rng(2).standard_normal(50) * 3])
    assert np.max(np.abs(oracle.act_grad(x, form) + oracle.act_grad(-x, form) - 1.0)) < 1e-14
    big = oracle.act_grad(np.array([-40.0, 40.0]), form)
    assert abs(big[0]) < 1e-12 and abs(big[1] - 1.0) < 1e-12


def _problem(seed, M=3, H=8, F=16, bias=True):
    r = _rng(seed)
    X = r.standard_normal((M, H))
    W1 = r.standard_normal((H, F)) * 0.4
    b1 = r.standard_normal(F) * 0.3 if bias else None
    W2 = r.standard_normal((F, H)) * 0.4
    dZ = r.standard_normal((M, H))
    return X, W1, b1, W2, dZ


def _loss(X, W1, b1, W2, dZ, T, i, form):
    # L_i = sum(dZ * Z_i): rank i's contribution, so its gradients are rank i's
    Y = oracle.colpar_act(X, W1, b1, T, i, form)
    return float(np.sum(dZ * oracle.rowpar_partial(Y, W2, T, i)))


@pytest.mark.parametrize("form", [TANH, ERF])
def test_backward_matches_finite_differences(form):
    X, W1, b1, W2, dZ = _problem(3)
    T, i = 2, 1
    g = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, T, i, form)
    Fs = W1.shape[1] // T
    h = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        up = _loss(X, W1, b1, W2, dZ, T, i, form)
        arr[idx] = old - h
        dn = _loss(X, W1, b1, W2, dZ, T, i, form)
        arr[idx] = old
        return (up - dn) / (2 * h)

    for idx in np.ndindex(*X.shape):
        assert abs(fd(X, idx) - g["dX_i"][idx]) < 1e-7
    for hh in range(W1.shape[0]):
        for c in range(Fs):
            assert abs(fd(W1, (hh, i * Fs + c)) - g["dW1_i"][hh, c]) < 1e-7
        # columns of other ranks do not touch rank i's output
        assert fd(W1, (hh, 0)) == 0.0
    for c in range(Fs):
        assert abs(fd(b1, (i * Fs + c,)) - g["db1_i"][c]) < 1e-7
        for hh in range(W2.shape[1]):
            assert abs(fd(W2, (i * Fs + c, hh)) - g["dW2_i"][c, hh]) < 1e-7


def test_backward_returns_the_forward_it_differentiates():
    X, W1, b1, W2, dZ = _problem(4)
    g = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, 2, 0, TANH)
    assert np.allclose(g["U_i"], oracle.colpar_linear(X, W1, b1, 2, 0), rtol=1e-14, atol=1e-14)
    assert np.allclose(g["Y_i"], oracle.colpar_gelu(X, W1, b1, 2, 0), rtol=1e-14, atol=1e-14)


def test_backward_identity_activation_is_exact_on_integers():
    # no activation: every gradient is an integer matrix product
    r = _rng(5)
    M, H, F, T, i = 4, 6, 8, 2, 1
    X = r.integers(-3, 4, (M, H)).astype(float)
    W1 = r.integers(-3, 4, (H, F)).astype(float)
    W2 = r.integers(-3, 4, (F, H)).astype(float)
    dZ = r.integers(-3, 4, (M, H)).astype(float)
    g = oracle.mlp_shard_bwd(X, W1, None, W2, dZ, T, i, NONE)
    Xi, W1i, W2i, dZi = (a.astype(np.int64) for a in (X, W1[:, 4:], W2[4:], dZ))
    dU = dZi @ W2i.T
    assert np.array_equal(g["dU_i"], dU)
    assert np.array_equal(g["dX_i"], dU @ W1i.T)
    assert np.array_equal(g["dW1_i"], Xi.T @ dU)
    assert np.array_equal(g["db1_i"], dU.sum(axis=0))
    assert np.array_equal(g["dW2_i"], (Xi @ W1i).T @ dZi)


@pytest.mark.parametrize("T", [2, 4])
def test_backward_shards_reassemble_the_unsharded_gradients(T):
    X, W1, b1, W2, dZ = _problem(6, M=5, H=8, F=16)
    full = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, 1, 0, ERF)
    parts = [oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, T, i, ERF) for i in range(T)]
    assert np.allclose(sum(p["dX_i"] for p in parts), full["dX_i"], rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.concatenate([p["dW1_i"] for p in parts], axis=1), full["dW1_i"])
    assert np.array_equal(np.concatenate([p["db1_i"] for p in parts]), full["db1_i"])
    assert np.array_equal(np.concatenate([p["dW2_i"] for p in parts], axis=0), full["dW2_i"])


def test_backward_linear_in_the_output_gradient():
    X, W1, b1, W2, dZ = _problem(7)
    dZ2 = _rng(8).standard_normal(dZ.shape)
    a = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, 2, 0, TANH)
    b = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ2, 2, 0, TANH)
    c = oracle.mlp_shard_bwd(X, W1, b1, W2, dZ - 3.0 * dZ2, 2, 0, TANH)
    for k in ("dX_i", "dW1_i", "db1_i", "dW2_i", "dU_i"):
        assert np.allclose(c[k], a[k] - 3.0 * b[k], rtol=1e-12, atol=1e-12)
    z = oracle.mlp_shard_bwd(X, W1, b1, W2, np.zeros_like(dZ), 2, 0, TANH)
    assert all(not np.any(z[k]) for k in ("dX_i", "dW1_i", "db1_i", "dW2_i"))


def test_backward_rejects_bad_arguments():
    X, W1, b1, W2, dZ = _problem(9)
    with pytest.raises(ValueError):
        oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, 3, 0)        # F % T
    with pytest.raises(ValueError):
        oracle.mlp_shard_bwd(X, W1, b1, W2, dZ, 2, 2)        # shard index
    with pytest.raises(ValueError):
        oracle.mlp_shard_bwd(X, W1, b1, W2, dZ[:, :4], 2, 0)  # dZ shape
    with pytest.raises(ValueError):
        oracle.act_grad(np.zeros(3), 7)
