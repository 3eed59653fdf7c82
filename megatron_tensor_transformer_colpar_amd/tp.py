"""ctypes binding of libtpcolpar.so: argument marshalling only.

The functions carry the C names and argument order of ``include/tp_colpar.h``.
Tensor arguments may be torch tensors (their ``data_ptr()`` is passed), plain
integer addresses, or None for NULL.  ``stream=None`` means torch's current
stream on the current device.  A non-OK status raises ``TPError`` carrying the
status and the library's message; the ``raw`` attribute exposes the C functions
for callers that want the status code itself.

Importing this module raises if the library has not been built: there is no
fallback path.

torch is imported before the library is opened: torch ships its own HIP
runtime under the same soname (libamdhip64.so.7), and the library must bind to
that one, or the process would hold two HIP runtimes that do not share devices,
memory or streams.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first; see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpcolpar.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libtpcolpar.so is not built (%s); build it with "
        "`python -m megatron_tensor_transformer_colpar_amd.build`" % LIB_PATH)


TP_OK, TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_UNSUPPORTED, TP_ERR_HIP, TP_ERR_ALIAS = range(6)
STATUS_NAMES = {0: "TP_OK", 1: "TP_ERR_NULL", 2: "TP_ERR_SHAPE", 3: "TP_ERR_UNSUPPORTED",
                4: "TP_ERR_HIP", 5: "TP_ERR_ALIAS"}
TP_BF16, TP_F32 = 0, 1
TP_GELU_TANH, TP_GELU_ERF = 0, 1
TP_REDUCE_RMS_BF16 = 1
TP_RMS_EPS = 1e-6
TP_MAX_T = 8
TP_NOALLOC_SCRATCH_BYTES = 16777216

_vp, _i64, _i32, _u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
_pp = ctypes.POINTER(_vp)


def _bind(lib):
    """Declare the C signatures of include/tp_colpar.h on a loaded build of the library."""
    lib.tp_colpar_gelu.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_rowpar_partial.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_shard_reduce.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _i64, _i64, _u32, _vp]
    lib.tp_mlp_shard_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_mlp_shard_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_colpar_gelu_group.argtypes = [_vp, _vp, _vp, _pp, _i64, _i64, _i64, _i32, _i32, _vp]
    lib.tp_rowpar_partial_group.argtypes = [_pp, _vp, _pp, _i64, _i64, _i64, _i32, _i32, _vp]
    lib.tp_mlp_group_fwd.argtypes = [_vp, _vp, _vp, _vp, _pp, _pp, _i64, _i64, _i64, _i32, _i32, _vp]
    lib.tp_layer_fwd.argtypes = [_vp, _vp, _pp, _vp, _i64, _vp, _vp, _vp, _pp, _pp, _i64, _i64, _i64, _i32, _vp]
    lib.tp_colpar_act.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp]
    lib.tp_colpar_gated.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp]
    lib.tp_colpar_linear.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_qkv_colpar.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                  _i32, _i32, _i32, _vp]
    lib.tp_attn_core.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i32,
                                 _vp, ctypes.c_size_t, _vp]
    lib.tp_attn_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i32]
    lib.tp_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.tp_colpar_act_train.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp]
    lib.tp_rowpar_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _u32, _vp]
    lib.tp_colpar_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _u32, _vp]
    lib.tp_mlp_shard_bwd.argtypes = [_vp] * 11 + [_i64, _i64, _i64, _i32, _i32, _i32, _u32, _vp]
    lib.tp_mlp_group_fwd_train.argtypes = [_vp, _vp, _vp, _pp, _pp, _i64, _i64, _i64, _i32, _i32, _vp]
    lib.tp_mlp_group_bwd.argtypes = [_vp, _vp, _vp, _pp, _pp, _vp, _pp, _pp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
                                     _u32, _vp]
    for _f in (lib.tp_colpar_gelu, lib.tp_rowpar_partial, lib.tp_shard_reduce, lib.tp_mlp_shard_fwd,
               lib.tp_mlp_shard_fwd_noalloc,
               lib.tp_colpar_gelu_group, lib.tp_rowpar_partial_group, lib.tp_mlp_group_fwd, lib.tp_layer_fwd,
               lib.tp_colpar_act, lib.tp_colpar_gated, lib.tp_colpar_linear, lib.tp_qkv_colpar, lib.tp_attn_core,
               lib.tp_colpar_act_train, lib.tp_rowpar_bwd, lib.tp_colpar_bwd, lib.tp_mlp_shard_bwd,
               lib.tp_mlp_group_fwd_train, lib.tp_mlp_group_bwd):
        _f.restype = ctypes.c_int
    lib.tp_last_error.argtypes = []
    lib.tp_last_error.restype = ctypes.c_char_p
    lib.tp_version.argtypes = []
    lib.tp_version.restype = ctypes.c_char_p
    return lib


raw = _bind(ctypes.CDLL(LIB_PATH))

EXPORTS = ("tp_colpar_gelu", "tp_rowpar_partial", "tp_shard_reduce", "tp_mlp_shard_fwd", "tp_mlp_shard_fwd_noalloc",
           "tp_colpar_gelu_group", "tp_rowpar_partial_group", "tp_mlp_group_fwd", "tp_layer_fwd",
           "tp_colpar_act", "tp_colpar_gated", "tp_colpar_linear", "tp_qkv_colpar", "tp_attn_core",
           "tp_attn_workspace_bytes", "tp_colpar_act_train", "tp_rowpar_bwd", "tp_colpar_bwd", "tp_mlp_shard_bwd",
           "tp_mlp_group_fwd_train", "tp_mlp_group_bwd", "tp_last_error", "tp_version")
TP_GRAD_ACCUMULATE = 1
TP_HEAD_DIM = 128


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int):
    if st != TP_OK:
        raise TPError(st, last_error())


def last_error() -> str:
    return raw.tp_last_error().decode()


def version() -> str:
    return raw.tp_version().decode()


def tp_colpar_gelu(X, W1t, b1, Y_i, M, H, F, T, i, dt=TP_BF16, stream=None):
    _check(raw.tp_colpar_gelu(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(Y_i), M, H, F, T, i, dt, _stream(stream)))


def tp_rowpar_partial(Y_i, W2t, Z_i, M, H, F, T, i, dt=TP_BF16, stream=None):
    _check(raw.tp_rowpar_partial(_ptr(Y_i), _ptr(W2t), _ptr(Z_i), M, H, F, T, i, dt, _stream(stream)))


def partial_array(partials):
    """Host array of device pointers (tp_shard_reduce, tp_mlp_group_fwd)."""
    return (_vp * len(partials))(*[_ptr(p) for p in partials])


def tp_shard_reduce(partials, T, residual, out_f32, out_bf16, M, H, flags=0, stream=None):
    arr = partials if isinstance(partials, ctypes.Array) else partial_array(partials)
    _check(raw.tp_shard_reduce(arr, T, _ptr(residual), _ptr(out_f32), _ptr(out_bf16), M, H, flags,
                               _stream(stream)))


def tp_mlp_shard_fwd(X, W1t, b1, W2t, Y_ws, Z_i, M, H, F, T, i, dt=TP_BF16, stream=None):
    _check(raw.tp_mlp_shard_fwd(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(W2t), _ptr(Y_ws), _ptr(Z_i), M, H, F,
                                T, i, dt, _stream(stream)))


def _arr(xs):
    return xs if isinstance(xs, ctypes.Array) else partial_array(xs)


def tp_mlp_shard_fwd_noalloc(X, W1t, b1, W2t, Z_i, M, H, F, T, i, dt=TP_BF16, stream=None):
    _check(raw.tp_mlp_shard_fwd_noalloc(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(W2t), _ptr(Z_i), M, H, F, T, i, dt,
                                        _stream(stream)))


def tp_colpar_gelu_group(X, W1t, b1, Y_ws, M, H, F, T, dt=TP_BF16, stream=None):
    _check(raw.tp_colpar_gelu_group(_ptr(X), _ptr(W1t), _ptr(b1), _arr(Y_ws), M, H, F, T, dt, _stream(stream)))


def tp_rowpar_partial_group(Y_ws, W2t, Z_parts, M, H, F, T, dt=TP_BF16, stream=None):
    _check(raw.tp_rowpar_partial_group(_arr(Y_ws), _ptr(W2t), _arr(Z_parts), M, H, F, T, dt, _stream(stream)))


def tp_mlp_group_fwd(X, W1t, b1, W2t, Y_ws, Z_parts, M, H, F, T, dt=TP_BF16, stream=None):
    _check(raw.tp_mlp_group_fwd(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(W2t), _arr(Y_ws), _arr(Z_parts), M, H, F, T,
                                dt, _stream(stream)))


def tp_colpar_act(X, W1t, b1, Y_i, M, H, F, T, i, act, dt=TP_BF16, stream=None):
    _check(raw.tp_colpar_act(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(Y_i), M, H, F, T, i, act, dt, _stream(stream)))


def tp_colpar_gated(X, Wgt, Wut, bg, bu, Y_i, M, H, F, T, i, act, dt=TP_BF16, stream=None):
    _check(raw.tp_colpar_gated(_ptr(X), _ptr(Wgt), _ptr(Wut), _ptr(bg), _ptr(bu), _ptr(Y_i), M, H, F, T, i, act,
                               dt, _stream(stream)))


def tp_layer_fwd(h, xhat, ctx, Wot, A, W1t, b1, W2t, Y_ws, parts, M, H, F, T, stream=None):
    _check(raw.tp_layer_fwd(_ptr(h), _ptr(xhat), _arr(ctx), _ptr(Wot), A, _ptr(W1t), _ptr(b1), _ptr(W2t),
                            _arr(Y_ws), _arr(parts), M, H, F, T, _stream(stream)))


def tp_colpar_linear(X, Wt, b, Y_i, ldy, M, H, N, T, i, dt=TP_BF16, stream=None):
    _check(raw.tp_colpar_linear(_ptr(X), _ptr(Wt), _ptr(b), _ptr(Y_i), ldy, M, H, N, T, i, dt, _stream(stream)))


def tp_qkv_colpar(X, Wq_t, Wk_t, Wv_t, bq, bk, bv, Q_i, ldq, K_i, V_i, ldkv, M, H, A, Akv, T, i, dt=TP_BF16,
                  stream=None):
    _check(raw.tp_qkv_colpar(_ptr(X), _ptr(Wq_t), _ptr(Wk_t), _ptr(Wv_t), _ptr(bq), _ptr(bk), _ptr(bv), _ptr(Q_i),
                             ldq, _ptr(K_i), _ptr(V_i), ldkv, M, H, A, Akv, T, i, dt, _stream(stream)))


def tp_attn_core(Q, K, V, ctx, kv_len, Bs, Sq, Lk, nh, nkv, d, ldq, ldkv, ldo, causal, workspace, ws_bytes,
                 stream=None):
    _check(raw.tp_attn_core(_ptr(Q), _ptr(K), _ptr(V), _ptr(ctx), _ptr(kv_len), Bs, Sq, Lk, nh, nkv, d, ldq, ldkv,
                            ldo, int(bool(causal)), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_attn_workspace_bytes(Bs, Sq, Lk, nh, nkv) -> int:
    return int(raw.tp_attn_workspace_bytes(Bs, Sq, Lk, nh, nkv))


def tp_colpar_act_train(X, W1t, b1, Y_i, U_i, M, H, F, T, i, act=TP_GELU_TANH, stream=None):
    _check(raw.tp_colpar_act_train(_ptr(X), _ptr(W1t), _ptr(b1), _ptr(Y_i), _ptr(U_i), M, H, F, T, i, act,
                                   _stream(stream)))


def tp_rowpar_bwd(dZ, W2t, Y_i, U_i, dU_i, dW2t, M, H, F, T, i, act=TP_GELU_TANH, flags=0, stream=None):
    _check(raw.tp_rowpar_bwd(_ptr(dZ), _ptr(W2t), _ptr(Y_i), _ptr(U_i), _ptr(dU_i), _ptr(dW2t), M, H, F, T, i, act,
                             flags, _stream(stream)))


def tp_colpar_bwd(X, W1t, dU_i, dX_i, dW1t, db1, M, H, F, T, i, flags=0, stream=None):
    _check(raw.tp_colpar_bwd(_ptr(X), _ptr(W1t), _ptr(dU_i), _ptr(dX_i), _ptr(dW1t), _ptr(db1), M, H, F, T, i, flags,
                             _stream(stream)))


def tp_mlp_shard_bwd(X, W1t, W2t, U_i, Y_i, dZ, dU_ws, dX_i, dW1t, db1, dW2t, M, H, F, T, i, act=TP_GELU_TANH,
                     flags=0, stream=None):
    _check(raw.tp_mlp_shard_bwd(_ptr(X), _ptr(W1t), _ptr(W2t), _ptr(U_i), _ptr(Y_i), _ptr(dZ), _ptr(dU_ws),
                                _ptr(dX_i), _ptr(dW1t), _ptr(db1), _ptr(dW2t), M, H, F, T, i, act, flags,
                                _stream(stream)))


def tp_mlp_group_fwd_train(X, W1t, b1, Y_ws, U_ws, M, H, F, T, act=TP_GELU_TANH, stream=None):
    _check(raw.tp_mlp_group_fwd_train(_ptr(X), _ptr(W1t), _ptr(b1), _arr(Y_ws), _arr(U_ws), M, H, F, T, act,
                                      _stream(stream)))


def tp_mlp_group_bwd(X, W1t, W2t, U_ws, Y_ws, dZ, dU_ws, dX_parts, dW1t, db1, dW2t, M, H, F, T, act=TP_GELU_TANH,
                     flags=0, stream=None):
    _check(raw.tp_mlp_group_bwd(_ptr(X), _ptr(W1t), _ptr(W2t), _arr(U_ws), _arr(Y_ws), _ptr(dZ), _arr(dU_ws),
                                _arr(dX_parts), _ptr(dW1t), _ptr(db1), _ptr(dW2t), M, H, F, T, act, flags,
                                _stream(stream)))
