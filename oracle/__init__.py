"""fp64 CPU oracle for one tensor-parallel rank's share of a Megatron MLP block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library: it is plain C (``oracle.c``) reached through ctypes, and
it takes the pages' logical matrices (``W1`` as [H, F], ``W2`` as [F, H]) as
float64 numpy arrays holding the exact values of the arrays the GPU receives.

Sources are cited per function in ``oracle.c``:
  * "Slice the matrix itself" (Tensor Parallelism scene): column split of the
    first MLP weight, row split of the second, the row-parallel summation.
  * "09. Tensor Parallelism in Action" section 1 (block split, pipeline
    diagram) and section 2 question 2 (GeLU commutes with the column split).
  * "Tensor parallelism" guide, "Concept" and "Walking through a transformer
    block" (column/row parallel, head-sharded attention, residual paths).
  * Vaswani et al., arXiv:1706.03762, section 3.2 (scaled dot-product and
    multi-head attention, the decoder's causal mask); Ainslie et al.,
    arXiv:2305.13245 (grouped key/value heads).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    i64, i32, dp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.orc_gelu.argtypes = [i64, dp, dp]
    lib.orc_gelu.restype = None
    lib.orc_colpar_gelu.argtypes = [i64, i64, i64, i32, i32, dp, dp, dp, dp]
    lib.orc_act.argtypes = [i32, i64, dp, dp]
    lib.orc_colpar_act.argtypes = [i64, i64, i64, i32, i32, i32, dp, dp, dp, dp]
    lib.orc_colpar_gated.argtypes = [i64, i64, i64, i32, i32, i32, dp, dp, dp, dp, dp, dp]
    lib.orc_rowpar_partial.argtypes = [i64, i64, i64, i32, i32, dp, dp, dp]
    lib.orc_shard_reduce.argtypes = [i32, i64, i64, dp, dp, dp, dp, ctypes.c_double]
    lib.orc_mlp_unsharded.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, dp]
    lib.orc_attention.argtypes = [i64, i64, i64, i32, i32, i32, i32, dp, dp, dp, dp, dp]
    lib.orc_act_grad.argtypes = [i32, i64, dp, dp]
    lib.orc_mlp_shard_bwd.argtypes = [i64, i64, i64, i32, i32, i32] + [dp] * 12
    for f in (lib.orc_colpar_gelu, lib.orc_rowpar_partial, lib.orc_shard_reduce,
              lib.orc_mlp_unsharded, lib.orc_act, lib.orc_colpar_act, lib.orc_colpar_gated,
              lib.orc_attention, lib.orc_act_grad, lib.orc_mlp_shard_bwd):
        f.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_set_threads.restype = None
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _bind(build())
    return _lib


@contextlib.contextmanager
def _swapped(path):
    """Test hook: route every call through another build of ``oracle.c``.

    Used only by the planted-mistake tests, which compile altered copies of the
    oracle and check that the pins reject them.
    """
    global _lib
    _load()
    with _lock:
        old, _lib = _lib, _bind(path)
    try:
        yield
    finally:
        with _lock:
            _lib = old


def _f64(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc, name):
    if rc != 0:
        raise ValueError("oracle: %s rejected its arguments" % name)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


def gelu(x):
    """GeLU, tanh form (Hendrycks & Gimpel), elementwise in fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().orc_gelu(x.size, _p(x), _p(y))
    return y


ACT_GELU_TANH, ACT_GELU_ERF, ACT_NONE = 0, 1, 2


def act(x, form: int):
    """Either GeLU form elementwise in fp64: ACT_GELU_TANH (tanh approximation)
    or ACT_GELU_ERF (exact x * Phi(x)); ACT_NONE is the identity."""
    x = _f64(x)
    y = np.empty_like(x)
    _check(_load().orc_act(int(form), x.size, _p(x), _p(y)), "act")
    return y


def colpar_act(X, W1, b1, T: int, i: int, form: int):
    """Shard i of T of the column-parallel up-projection with the chosen GeLU form."""
    X = _f64(X)
    M, H = X.shape
    W1 = _f64(W1)
    if W1.shape[0] != H:
        raise ValueError("oracle: W1 must be [H, F]")
    F = W1.shape[1]
    b1 = None if b1 is None else _f64(b1, (F,))
    if F % T:
        raise ValueError("oracle: F % T != 0")
    Y = np.empty((M, F // T))
    _check(_load().orc_colpar_act(M, H, F, T, i, int(form), _p(X), _p(W1), _p(b1), _p(Y)), "colpar_act")
    return Y


def act_grad(x, form: int):
    """Derivative of either GeLU form (or of the identity), elementwise in fp64."""
    x = _f64(x)
    y = np.empty_like(x)
    _check(_load().orc_act_grad(int(form), x.size, _p(x), _p(y)), "act_grad")
    return y


def mlp_shard_bwd(X, W1, b1, W2, dZ, T: int, i: int, form: int = ACT_GELU_TANH):
    """Backward pass of rank i's MLP share for the output gradient dZ [M, H].

    Returns a dict: dX_i [M,H] (a partial; dX = sum over ranks), dW1_i [H,Fs]
    (columns C_i of dW1), db1_i [Fs], dW2_i [Fs,H] (rows C_i of dW2), and the
    forward's U_i, Y_i and the GeLU-input gradient dU_i [M,Fs].
    """
    X = _f64(X)
    M, H = X.shape
    W1 = _f64(W1)
    if W1.shape[0] != H:
        raise ValueError("oracle: W1 must be [H, F]")
    F = W1.shape[1]
    W2 = _f64(W2, (F, H))
    b1 = None if b1 is None else _f64(b1, (F,))
    dZ = _f64(dZ, (M, H))
    if F % T:
        raise ValueError("oracle: F % T != 0")
    Fs = F // T
    out = {k: np.empty(s) for k, s in (("dX_i", (M, H)), ("dW1_i", (H, Fs)), ("db1_i", (Fs,)), ("dW2_i", (Fs, H)),
                                       ("U_i", (M, Fs)), ("Y_i", (M, Fs)), ("dU_i", (M, Fs)))}
    _check(_load().orc_mlp_shard_bwd(M, H, F, T, i, int(form), _p(X), _p(W1), _p(b1), _p(W2), _p(dZ),
                                     _p(out["dX_i"]), _p(out["dW1_i"]), _p(out["db1_i"]), _p(out["dW2_i"]),
                                     _p(out["U_i"]), _p(out["Y_i"]), _p(out["dU_i"])), "mlp_shard_bwd")
    return out


def colpar_linear(X, W, b, T: int, i: int):
    """Shard i of T of a column-parallel projection with no activation:
    X W[:, C_i] + b[C_i] (the attention's query, key and value projections)."""
    return colpar_act(X, W, b, T, i, ACT_NONE)


def attention(Q, K, V, nh: int, nkv: int, causal: bool, kv_len=None):
    """Scaled dot-product attention of nh query heads over nkv key/value heads.

    Q [Bs, Sq, nh*d], K and V [Bs, Lk, nkv*d]; kv_len: valid keys per sequence
    (default Lk).  Query s of sequence b sits at position kv_len[b] - Sq + s;
    causal attention sees keys up to that position.  Returns ctx [Bs, Sq, nh*d].
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    if Q.ndim != 3 or K.ndim != 3 or K.shape != V.shape or K.shape[0] != Q.shape[0]:
        raise ValueError("oracle: Q [Bs,Sq,nh*d], K and V [Bs,Lk,nkv*d]")
    Bs, Sq, qw = Q.shape
    Lk, kw = K.shape[1], K.shape[2]
    if qw % nh or kw % nkv or qw // nh != kw // nkv:
        raise ValueError("oracle: head widths of Q and K/V differ")
    d = qw // nh
    lens = None if kv_len is None else np.ascontiguousarray(kv_len, dtype=np.int64)
    if lens is not None and lens.shape != (Bs,):
        raise ValueError("oracle: kv_len must have one entry per sequence")
    ctx = np.empty((Bs, Sq, qw))
    _check(_load().orc_attention(Bs, Sq, Lk, nh, nkv, d, int(bool(causal)), _p(lens), _p(Q), _p(K), _p(V),
                                 _p(ctx)), "attention")
    return ctx


def colpar_gated(X, Wg, Wu, bg, bu, T: int, i: int, form: int):
    """Shard i of T of the gated first layer ("Gate/Up"):
    a(X Wg[:, C_i] + bg[C_i]) * (X Wu[:, C_i] + bu[C_i]), a the chosen GeLU form."""
    X = _f64(X)
    M, H = X.shape
    Wg, Wu = _f64(Wg), _f64(Wu)
    if Wg.shape[0] != H or Wu.shape != Wg.shape:
        raise ValueError("oracle: Wg and Wu must both be [H, F]")
    F = Wg.shape[1]
    bg = None if bg is None else _f64(bg, (F,))
    bu = None if bu is None else _f64(bu, (F,))
    if F % T:
        raise ValueError("oracle: F % T != 0")
    Y = np.empty((M, F // T))
    _check(_load().orc_colpar_gated(M, H, F, T, i, int(form), _p(X), _p(Wg), _p(Wu), _p(bg), _p(bu), _p(Y)),
           "colpar_gated")
    return Y


def colpar_gelu(X, W1, b1, T: int, i: int):
    """Shard i of T of the column-parallel up-projection: g(X W1[:, C_i] + b1[C_i])."""
    X = _f64(X)
    M, H = X.shape
    W1 = _f64(W1)
    if W1.shape[0] != H:
        raise ValueError("oracle: W1 must be [H, F]")
    F = W1.shape[1]
    b1 = None if b1 is None else _f64(b1, (F,))
    if F % T:
        raise ValueError("oracle: F % T != 0")
    Y = np.empty((M, F // T))
    _check(_load().orc_colpar_gelu(M, H, F, T, i, _p(X), _p(W1), _p(b1), _p(Y)), "colpar_gelu")
    return Y


def rowpar_partial(Y_i, W2, T: int, i: int):
    """Shard i of T of the row-parallel down-projection: Y_i W2[C_i, :] (a partial sum)."""
    W2 = _f64(W2)
    F, H = W2.shape
    if F % T:
        raise ValueError("oracle: F % T != 0")
    Y_i = _f64(Y_i)
    if Y_i.ndim != 2 or Y_i.shape[1] != F // T:
        raise ValueError("oracle: Y_i must be [M, F/T]")
    M = Y_i.shape[0]
    Z = np.empty((M, H))
    _check(_load().orc_rowpar_partial(M, H, F, T, i, _p(Y_i), _p(W2), _p(Z)), "rowpar_partial")
    return Z


def shard_reduce(partials, residual=None, rms_eps=None):
    """Sum of T partials [T, M, H] (+ residual [M, H]).

    Returns ``out`` or, when ``rms_eps`` is given, ``(out, out / rms(out))``.
    """
    P = _f64(partials)
    T, M, H = P.shape
    R = None if residual is None else _f64(residual, (M, H))
    out = np.empty((M, H))
    rms = np.empty((M, H)) if rms_eps is not None else None
    eps = 0.0 if rms_eps is None else float(rms_eps)
    _check(_load().orc_shard_reduce(T, M, H, _p(P), _p(R), _p(out), _p(rms), eps), "shard_reduce")
    return out if rms is None else (out, rms)


def mlp_unsharded(X, W1, b1, W2):
    """The unsharded block the shards reconstruct: returns (Y, Z), Y = g(X W1 + b1), Z = Y W2."""
    X = _f64(X)
    M, H = X.shape
    W1 = _f64(W1)
    F = W1.shape[1]
    W2 = _f64(W2, (F, H))
    b1 = None if b1 is None else _f64(b1, (F,))
    Y = np.empty((M, F))
    Z = np.empty((M, H))
    _check(_load().orc_mlp_unsharded(M, H, F, _p(X), _p(W1), _p(b1), _p(W2), _p(Y), _p(Z)),
           "mlp_unsharded")
    return Y, Z


def mlp_shard(X, W1, b1, W2, T: int, i: int):
    """Rank i's share: (Y_i, Z_i) with Z_i its row-parallel partial."""
    Y_i = colpar_gelu(X, W1, b1, T, i)
    return Y_i, rowpar_partial(Y_i, W2, T, i)


def layer_fwd(h, ctx_shards, Wo, W1, b1, W2, T: int, eps: float):
    """One block of the layer stack on the residual stream h [M, H] (fp64).

    Both all-reduces sit on residual paths ("Tensor parallelism" guide,
    "Walking through a transformer block"); one follows the head-sharded
    attention output projection, one the MLP ("Slice the matrix itself",
    "All-Reduce Synchronization"):
      h  <- h + sum_i ctx_i . Wo[A_i, :]          (attention out-projection)
      xh <- h / rms(h)   (row RMS with eps; not from the pages: it keeps a deep
                          stack with no normalisation layer finite)
      h  <- h + sum_i GeLU(xh . W1[:, C_i] + b1[C_i]) . W2[C_i, :]
    ctx_shards: T arrays [M, A/T] (rank i's heads); Wo [A, H]; W1 [H, F];
    W2 [F, H].  Returns (h_out, xh).
    """
    P = np.stack([rowpar_partial(ctx_shards[i], Wo, T, i) for i in range(T)])
    h1, xh = shard_reduce(P, h, rms_eps=eps)
    Z = np.stack([mlp_shard(xh, W1, b1, W2, T, i)[1] for i in range(T)])
    return shard_reduce(Z, h1), xh
