"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and every invalid argument is rejected with the documented
status before any HIP call (so these run on a machine without a GPU).
"""
import ctypes
import os
import re

import pytest

from megatron_tensor_transformer_colpar_amd import tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_colpar.h")

BF16, F32 = tp.TP_BF16, tp.TP_F32
# Fake, 16-byte aligned device addresses far apart: validation never
# dereferences them and a rejected call makes no HIP call.
P = [0x10000000 * (k + 1) for k in range(12)]


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:tp_status|const char \*|size_t)\s*(tp_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(tp.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_empty_error():
    assert "gfx950" in tp.version()


def colpar(X=P[0], W=P[1], b=P[2], Y=P[3], M=4, H=64, F=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_colpar_gelu(X, W, b, Y, M, H, F, T, i, dt, None)


def rowpar(Y=P[3], W=P[4], Z=P[5], M=4, H=64, F=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_rowpar_partial(Y, W, Z, M, H, F, T, i, dt, None)


def mlp(X=P[0], W1=P[1], b=P[2], W2=P[4], Y=P[3], Z=P[5], M=4, H=64, F=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_mlp_shard_fwd(X, W1, b, W2, Y, Z, M, H, F, T, i, dt, None)


def reduce(parts=None, T=2, res=None, out=P[8], ob=None, M=4, H=64, flags=0):
    parts = [P[6], P[7]] if parts is None else parts
    arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts else None
    return tp.raw.tp_shard_reduce(arr, T, res, out, ob, M, H, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), tp.TP_ERR_SHAPE),
    (dict(M=2**31), tp.TP_ERR_SHAPE),
    (dict(H=0), tp.TP_ERR_SHAPE),
    (dict(F=0), tp.TP_ERR_SHAPE),
    (dict(T=0), tp.TP_ERR_SHAPE),
    (dict(T=9, F=64 * 9), tp.TP_ERR_SHAPE),
    (dict(F=250), tp.TP_ERR_SHAPE),
    (dict(i=-1), tp.TP_ERR_SHAPE),
    (dict(i=4), tp.TP_ERR_SHAPE),
    (dict(X=None), tp.TP_ERR_NULL),
    (dict(W=None), tp.TP_ERR_NULL),
    (dict(Y=None), tp.TP_ERR_NULL),
    (dict(dt=7), tp.TP_ERR_UNSUPPORTED),
    (dict(H=96), tp.TP_ERR_UNSUPPORTED),
    (dict(F=4 * 96), tp.TP_ERR_UNSUPPORTED),
    (dict(H=2**23), tp.TP_ERR_UNSUPPORTED),
    (dict(X=P[0] + 8), tp.TP_ERR_UNSUPPORTED),
    (dict(b=P[2] + 2), tp.TP_ERR_UNSUPPORTED),
    (dict(Y=P[0] + 64), tp.TP_ERR_ALIAS),
    (dict(Y=P[1] + 4096), tp.TP_ERR_ALIAS),
])
def test_colpar_rejects(kw, status):
    assert colpar(**kw) == status
    assert "tp_colpar_gelu" in tp.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(M=-5), tp.TP_ERR_SHAPE),
    (dict(T=3), tp.TP_ERR_SHAPE),          # 256 % 3
    (dict(i=7), tp.TP_ERR_SHAPE),
    (dict(Z=None), tp.TP_ERR_NULL),
    (dict(W=None), tp.TP_ERR_NULL),
    (dict(dt=2), tp.TP_ERR_UNSUPPORTED),
    (dict(Z=P[5] + 4), tp.TP_ERR_UNSUPPORTED),
    (dict(Z=P[3]), tp.TP_ERR_ALIAS),
    (dict(Z=P[4] + 1024), tp.TP_ERR_ALIAS),
])
def test_rowpar_rejects(kw, status):
    assert rowpar(**kw) == status
    assert "tp_rowpar_partial" in tp.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(Y=None), tp.TP_ERR_NULL),
    (dict(W2=None), tp.TP_ERR_NULL),
    (dict(Z=P[0]), tp.TP_ERR_ALIAS),        # Z over X
    (dict(Z=P[2]), tp.TP_ERR_ALIAS),        # Z over b1
    (dict(Y=P[4]), tp.TP_ERR_ALIAS),        # workspace over W2t
    (dict(Y=P[5]), tp.TP_ERR_ALIAS),        # workspace over Z
])
def test_mlp_shard_rejects(kw, status):
    assert mlp(**kw) == status
    assert "tp_mlp_shard_fwd" in tp.last_error()


def mlp_noalloc(X=P[0], W1=P[1], b=P[2], W2=P[4], Z=P[5], M=4, H=64, F=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_mlp_shard_fwd_noalloc(X, W1, b, W2, Z, M, H, F, T, i, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), tp.TP_ERR_NULL),
    (dict(W1=None), tp.TP_ERR_NULL),
    (dict(W2=None), tp.TP_ERR_NULL),
    (dict(Z=None), tp.TP_ERR_NULL),
    (dict(T=3), tp.TP_ERR_SHAPE),
    (dict(i=4), tp.TP_ERR_SHAPE),
    (dict(H=96), tp.TP_ERR_UNSUPPORTED),
    (dict(Z=P[5] + 4), tp.TP_ERR_UNSUPPORTED),
    # the staging limit: 4096 x 4096 bf16 is 32 MiB, 2 x the 16 MiB buffer
    (dict(M=4096, H=64, F=4096, T=1), tp.TP_ERR_UNSUPPORTED),
    (dict(M=2049, H=64, F=16384, T=4), tp.TP_ERR_UNSUPPORTED),
    (dict(M=1025, H=64, F=4096, T=1, dt=F32), tp.TP_ERR_UNSUPPORTED),
    (dict(Z=P[0]), tp.TP_ERR_ALIAS),        # Z over X
    (dict(Z=P[4] + 256), tp.TP_ERR_ALIAS),  # Z over W2t
])
def test_mlp_noalloc_rejects(kw, status):
    assert mlp_noalloc(**kw) == status
    assert "tp_mlp_shard_fwd_noalloc" in tp.last_error()
    if kw.get("M", 0) >= 1024:
        assert "limit" in tp.last_error()


def test_mlp_noalloc_limit_and_empty_call():
    assert tp.TP_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert mlp_noalloc(M=0) == tp.TP_OK


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), tp.TP_ERR_SHAPE),
    (dict(T=9, parts=[P[6]] * 9), tp.TP_ERR_SHAPE),
    (dict(M=-1), tp.TP_ERR_SHAPE),
    (dict(H=0), tp.TP_ERR_SHAPE),
    (dict(parts=[], T=2), tp.TP_ERR_NULL),
    (dict(parts=[P[6], None]), tp.TP_ERR_NULL),
    (dict(out=None), tp.TP_ERR_NULL),
    (dict(flags=1), tp.TP_ERR_NULL),         # RMS copy needs out_bf16
    (dict(flags=2, ob=P[9]), tp.TP_ERR_UNSUPPORTED),
    (dict(H=66), tp.TP_ERR_UNSUPPORTED),
    (dict(out=P[8] + 4), tp.TP_ERR_UNSUPPORTED),
    (dict(parts=[P[6], P[7] + 8]), tp.TP_ERR_UNSUPPORTED),
    (dict(out=P[6]), tp.TP_ERR_ALIAS),
    (dict(ob=P[7] + 128), tp.TP_ERR_ALIAS),
    (dict(ob=P[8]), tp.TP_ERR_ALIAS),
    (dict(res=P[8] + 256), tp.TP_ERR_ALIAS),
])
def test_reduce_rejects(kw, status):
    assert reduce(**kw) == status
    assert "tp_shard_reduce" in tp.last_error()


def test_empty_calls_are_ok_and_touch_nothing():
    # M == 0 is a valid empty call: TP_OK without any HIP call, so it works
    # here with fake pointers and no GPU.
    assert colpar(M=0) == tp.TP_OK
    assert rowpar(M=0) == tp.TP_OK
    assert mlp(M=0) == tp.TP_OK
    assert reduce(M=0) == tp.TP_OK
    assert reduce(M=0, res=P[8], flags=1, ob=P[9]) == tp.TP_OK   # in-place residual allowed
    assert tp.last_error() == ""


def test_binding_raises_with_status_and_message():
    with pytest.raises(tp.TPError) as e:
        tp.tp_colpar_gelu(P[0], P[1], P[2], P[3], 4, 64, 250, 4, 0, BF16, stream=0)
    assert e.value.status == tp.TP_ERR_SHAPE and "divisible" in str(e.value)


def test_one_hip_runtime_in_the_process():
    # The binding opens the library after torch, so the library binds to the
    # HIP runtime torch already loaded instead of loading a second one.
    maps = open("/proc/self/maps").read()
    libs = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(libs) == 1, libs


def arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def group(X=P[0], W1=P[1], b=P[2], W2=P[4], Y=None, Z=None, M=4, H=64, F=256, T=2, dt=BF16):
    Y = arr(P[6], P[7]) if Y is None else Y
    Z = arr(P[8], P[9]) if Z is None else Z
    return tp.raw.tp_mlp_group_fwd(X, W1, b, W2, Y, Z, M, H, F, T, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=3), tp.TP_ERR_SHAPE),
    (dict(X=None), tp.TP_ERR_NULL),
    (dict(W2=None), tp.TP_ERR_NULL),
    (dict(Y=arr(P[6], None)), tp.TP_ERR_NULL),
    (dict(Z=arr(None, P[9])), tp.TP_ERR_NULL),
    (dict(Y=arr(P[6], P[7] + 4)), tp.TP_ERR_UNSUPPORTED),
    (dict(Y=arr(P[6], P[6] + 256)), tp.TP_ERR_ALIAS),     # two shards' Y overlap
    (dict(Z=arr(P[8], P[6])), tp.TP_ERR_ALIAS),           # Z over a Y
    (dict(Z=arr(P[0], P[9])), tp.TP_ERR_ALIAS),           # Z over X
    (dict(Y=arr(P[4] + 64, P[7])), tp.TP_ERR_ALIAS),      # Y over W2t
])
def test_group_rejects(kw, status):
    assert group(**kw) == status
    assert "tp_mlp_group_fwd" in tp.last_error()


def test_group_halves_reject_and_accept_empty():
    Y, Z = arr(P[6], P[7]), arr(P[8], P[9])
    assert tp.raw.tp_colpar_gelu_group(P[0], None, None, Y, 4, 64, 256, 2, BF16, None) == tp.TP_ERR_NULL
    assert tp.raw.tp_rowpar_partial_group(Y, P[4], None, 4, 64, 256, 2, BF16, None) == tp.TP_ERR_NULL
    assert tp.raw.tp_colpar_gelu_group(P[0], P[1], P[2], Y, 0, 64, 256, 2, BF16, None) == tp.TP_OK
    assert tp.raw.tp_rowpar_partial_group(Y, P[4], Z, 0, 64, 256, 2, BF16, None) == tp.TP_OK
    assert group(M=0) == tp.TP_OK


def layer(h=P[10], xh=P[11], ctx=None, Wo=P[1], A=256, W1=P[2], b=P[3], W2=P[4], Y=None, parts=None,
          M=4, H=64, F=256, T=2):
    ctx = arr(P[5], P[5] + 0x100000) if ctx is None else ctx
    Y = arr(P[6], P[7]) if Y is None else Y
    parts = arr(P[8], P[9]) if parts is None else parts
    return tp.raw.tp_layer_fwd(h, xh, ctx, Wo, A, W1, b, W2, Y, parts, M, H, F, T, None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), tp.TP_ERR_NULL),
    (dict(xh=None), tp.TP_ERR_NULL),
    (dict(ctx=arr(P[5], None)), tp.TP_ERR_NULL),
    (dict(Wo=None), tp.TP_ERR_NULL),
    (dict(A=255), tp.TP_ERR_SHAPE),
    (dict(A=2 * 96), tp.TP_ERR_UNSUPPORTED),
    (dict(h=P[10] + 8), tp.TP_ERR_UNSUPPORTED),
    (dict(xh=P[10] + 64), tp.TP_ERR_ALIAS),           # xhat over h
    (dict(h=P[8]), tp.TP_ERR_ALIAS),                  # h over a partial
    (dict(parts=arr(P[8], P[5])), tp.TP_ERR_ALIAS),   # partial over ctx
])
def test_layer_rejects(kw, status):
    assert layer(**kw) == status
    assert "tp_layer_fwd" in tp.last_error()


def test_layer_empty_is_ok():
    assert layer(M=0) == tp.TP_OK


# ------------------------------------- GeLU form choice and gated first layer
def colpar_act(X=P[0], W=P[1], b=P[2], Y=P[3], M=4, H=64, F=256, T=4, i=0, act=tp.TP_GELU_ERF, dt=BF16):
    return tp.raw.tp_colpar_act(X, W, b, Y, M, H, F, T, i, act, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), tp.TP_ERR_SHAPE),
    (dict(i=4), tp.TP_ERR_SHAPE),
    (dict(X=None), tp.TP_ERR_NULL),
    (dict(act=2), tp.TP_ERR_UNSUPPORTED),
    (dict(act=-1), tp.TP_ERR_UNSUPPORTED),
    (dict(H=96), tp.TP_ERR_UNSUPPORTED),
    (dict(Y=P[0] + 64), tp.TP_ERR_ALIAS),
])
def test_colpar_act_rejects(kw, status):
    assert colpar_act(**kw) == status
    assert "tp_colpar_act" in tp.last_error()


def gated(X=P[0], Wg=P[1], Wu=P[4], bg=P[2], bu=P[5], Y=P[3], M=4, H=64, F=256, T=4, i=0,
          act=tp.TP_GELU_TANH, dt=BF16):
    return tp.raw.tp_colpar_gated(X, Wg, Wu, bg, bu, Y, M, H, F, T, i, act, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=3), tp.TP_ERR_SHAPE),
    (dict(i=-1), tp.TP_ERR_SHAPE),
    (dict(X=None), tp.TP_ERR_NULL),
    (dict(Wg=None), tp.TP_ERR_NULL),
    (dict(Wu=None), tp.TP_ERR_NULL),
    (dict(Y=None), tp.TP_ERR_NULL),
    (dict(act=5), tp.TP_ERR_UNSUPPORTED),
    (dict(dt=3), tp.TP_ERR_UNSUPPORTED),
    (dict(F=4 * 96), tp.TP_ERR_UNSUPPORTED),
    (dict(Wu=P[4] + 8), tp.TP_ERR_UNSUPPORTED),
    (dict(bu=P[5] + 2), tp.TP_ERR_UNSUPPORTED),
    (dict(Y=P[1] + 4096), tp.TP_ERR_ALIAS),      # Y over the gate weights
    (dict(Y=P[4] + 4096), tp.TP_ERR_ALIAS),      # Y over the up weights
    (dict(Y=P[5]), tp.TP_ERR_ALIAS),             # Y over the up bias
])
def test_colpar_gated_rejects(kw, status):
    assert gated(**kw) == status
    assert "tp_colpar_gated" in tp.last_error()


def test_variant_empty_calls_are_ok():
    assert colpar_act(M=0) == tp.TP_OK
    assert gated(M=0) == tp.TP_OK
    assert gated(M=0, bg=None, bu=None, act=tp.TP_GELU_ERF) == tp.TP_OK
    assert tp.last_error() == ""


# ------------------------------------------------ attention front half
def linear(X=P[0], W=P[1], b=P[2], Y=P[3], ldy=64, M=4, H=64, N=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_colpar_linear(X, W, b, Y, ldy, M, H, N, T, i, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), tp.TP_ERR_SHAPE),
    (dict(T=3), tp.TP_ERR_SHAPE),
    (dict(ldy=56), tp.TP_ERR_SHAPE),          # below N/T
    (dict(W=None), tp.TP_ERR_NULL),
    (dict(Y=None), tp.TP_ERR_NULL),
    (dict(ldy=68), tp.TP_ERR_UNSUPPORTED),    # not a multiple of 8
    (dict(H=96), tp.TP_ERR_UNSUPPORTED),
    (dict(b=P[2] + 4), tp.TP_ERR_UNSUPPORTED),
    (dict(Y=P[1] + 64), tp.TP_ERR_ALIAS),     # Y over the weight
    (dict(Y=P[0] + 2, X=P[0]), tp.TP_ERR_UNSUPPORTED),
])
def test_colpar_linear_rejects(kw, status):
    assert linear(**kw) == status
    assert "tp_colpar_linear" in tp.last_error()


def qkv(X=P[0], Wq=P[1], Wk=P[2], Wv=P[3], bq=P[4], bk=P[5], bv=P[6], Q=P[7], ldq=64, K=P[8], V=P[9], ldkv=64,
        M=4, H=64, A=256, Akv=256, T=4, i=0, dt=BF16):
    return tp.raw.tp_qkv_colpar(X, Wq, Wk, Wv, bq, bk, bv, Q, ldq, K, V, ldkv, M, H, A, Akv, T, i, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(i=4), tp.TP_ERR_SHAPE),
    (dict(Akv=202), tp.TP_ERR_SHAPE),         # not divisible by T
    (dict(Akv=200), tp.TP_ERR_UNSUPPORTED),   # Akv/T not a multiple of 64
    (dict(Wk=None), tp.TP_ERR_NULL),
    (dict(V=None), tp.TP_ERR_NULL),
    (dict(ldkv=60), tp.TP_ERR_SHAPE),
    (dict(K=P[7] + 128), tp.TP_ERR_ALIAS),    # K over Q
    (dict(V=P[8]), tp.TP_ERR_ALIAS),          # V over K
    (dict(Q=P[3] + 256), tp.TP_ERR_ALIAS),    # Q over Wv
])
def test_qkv_rejects(kw, status):
    assert qkv(**kw) == status
    assert "tp_qkv_colpar" in tp.last_error()


def attn(Q=P[0], K=P[1], V=P[2], ctx=P[3], kv_len=None, Bs=2, Sq=256, Lk=256, nh=8, nkv=8, d=128, ldq=1024,
         ldkv=1024, ldo=1024, causal=1, ws=None, ws_bytes=0):
    return tp.raw.tp_attn_core(Q, K, V, ctx, kv_len, Bs, Sq, Lk, nh, nkv, d, ldq, ldkv, ldo, causal, ws, ws_bytes,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(Bs=-1), tp.TP_ERR_SHAPE),
    (dict(Lk=0), tp.TP_ERR_SHAPE),
    (dict(nkv=3), tp.TP_ERR_SHAPE),           # nh % nkv
    (dict(Sq=300), tp.TP_ERR_SHAPE),          # causal, more queries than keys
    (dict(ldq=1000), tp.TP_ERR_SHAPE),        # below nh * 128
    (dict(ldkv=512), tp.TP_ERR_SHAPE),
    (dict(Q=None), tp.TP_ERR_NULL),
    (dict(ctx=None), tp.TP_ERR_NULL),
    (dict(d=64), tp.TP_ERR_UNSUPPORTED),
    (dict(ldo=1028), tp.TP_ERR_UNSUPPORTED),  # not a multiple of 8
    (dict(K=P[1] + 8), tp.TP_ERR_UNSUPPORTED),
    (dict(kv_len=P[4] + 2), tp.TP_ERR_UNSUPPORTED),
    (dict(Sq=1, Lk=1 << 20), tp.TP_ERR_UNSUPPORTED),   # rows beyond 32-bit offsets
    (dict(Sq=1), tp.TP_ERR_NULL),             # the split-key path needs a workspace
    (dict(Sq=1, ws=P[5], ws_bytes=16), tp.TP_ERR_SHAPE),
    (dict(ctx=P[0] + 2048), tp.TP_ERR_ALIAS),
    (dict(Sq=1, ws=P[1] + 4096, ws_bytes=1 << 20), tp.TP_ERR_ALIAS),
])
def test_attn_core_rejects(kw, status):
    assert attn(**kw) == status
    assert "tp_attn_core" in tp.last_error()


def test_attn_workspace_bytes():
    # prefill shapes need none; the split-key decode path needs its partials
    assert tp.tp_attn_workspace_bytes(4, 2048, 2048, 8, 8) == 0
    n = tp.tp_attn_workspace_bytes(8, 1, 2048, 8, 8)
    # 4096 arrival counters (16 KiB), then the partials of 8 x 8 query rows
    # (128 weighted dims, max and sum) per chunk
    assert n > 16384 and (n - 16384) % (8 * 8 * 130 * 4) == 0
    # more (sequence, key/value head) pairs than counters: the prefill kernel, no workspace
    assert tp.tp_attn_workspace_bytes(512, 1, 2048, 8, 8) > 0
    assert tp.tp_attn_workspace_bytes(513, 1, 2048, 8, 8) == 0
    assert tp.tp_attn_workspace_bytes(0, 1, 2048, 8, 8) == 0
    assert tp.tp_attn_workspace_bytes(1, 1, 2048, 8, 3) == 0     # invalid grouping
    assert attn(Bs=8, Sq=1, Lk=2048, ws=P[5], ws_bytes=n - 4) == tp.TP_ERR_SHAPE


def test_attention_empty_calls_are_ok():
    assert linear(M=0) == tp.TP_OK
    assert qkv(M=0) == tp.TP_OK
    assert attn(Bs=0) == tp.TP_OK
    assert attn(Sq=0, causal=0) == tp.TP_OK
    assert tp.last_error() == ""


# ------------------------------------------------------------ backward pass
def rowpar_bwd(dZ=P[0], W2t=P[1], Y=P[2], U=P[3], dU=P[4], dW2t=P[5], M=4, H=64, F=256, T=4, i=0,
               act=tp.TP_GELU_TANH, flags=0):
    return tp.raw.tp_rowpar_bwd(dZ, W2t, Y, U, dU, dW2t, M, H, F, T, i, act, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), tp.TP_ERR_SHAPE),
    (dict(i=4), tp.TP_ERR_SHAPE),
    (dict(dZ=None), tp.TP_ERR_NULL),
    (dict(dU=None), tp.TP_ERR_NULL),
    (dict(Y=None), tp.TP_ERR_NULL),          # the weight gradient needs Y_i
    (dict(act=9), tp.TP_ERR_UNSUPPORTED),
    (dict(flags=2), tp.TP_ERR_UNSUPPORTED),
    (dict(H=96), tp.TP_ERR_UNSUPPORTED),
    (dict(M=1 << 20, H=4096, F=4096, T=1), tp.TP_ERR_UNSUPPORTED),   # 32-bit offsets
    (dict(dW2t=P[5] + 4), tp.TP_ERR_UNSUPPORTED),
    (dict(dU=P[2]), tp.TP_ERR_ALIAS),        # dU over Y_i
    (dict(dW2t=P[1]), tp.TP_ERR_ALIAS),      # dW2 over W2
])
def test_rowpar_bwd_rejects(kw, status):
    assert rowpar_bwd(**kw) == status
    assert "tp_rowpar_bwd" in tp.last_error()


def colpar_bwd(X=P[0], W1t=P[1], dU=P[2], dX=P[3], dW1t=P[4], db1=P[5], M=4, H=64, F=256, T=4, i=1, flags=0):
    return tp.raw.tp_colpar_bwd(X, W1t, dU, dX, dW1t, db1, M, H, F, T, i, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=3), tp.TP_ERR_SHAPE),
    (dict(dU=None), tp.TP_ERR_NULL),
    (dict(W1t=None), tp.TP_ERR_NULL),        # dX needs W1t
    (dict(X=None), tp.TP_ERR_NULL),          # dW1 needs X
    (dict(flags=8), tp.TP_ERR_UNSUPPORTED),
    (dict(db1=P[5] + 8), tp.TP_ERR_UNSUPPORTED),
    (dict(dX=P[2]), tp.TP_ERR_ALIAS),        # dX over dU
    (dict(db1=P[4] + 64), tp.TP_ERR_ALIAS),  # db1 inside dW1
])
def test_colpar_bwd_rejects(kw, status):
    assert colpar_bwd(**kw) == status
    assert "tp_colpar_bwd" in tp.last_error()


def test_backward_optional_outputs_and_empty_calls():
    assert colpar_bwd(M=0) == tp.TP_OK
    assert rowpar_bwd(M=0) == tp.TP_OK
    # without the outputs that need them, X / W1t / Y_i may be NULL (M = 0: nothing launched)
    assert colpar_bwd(X=None, W1t=None, dX=None, dW1t=None, M=0) == tp.TP_OK
    assert rowpar_bwd(Y=None, dW2t=None, U=None, M=0) == tp.TP_OK
    assert tp.raw.tp_colpar_act_train(P[0], P[1], P[2], P[3], P[4], 0, 64, 256, 4, 0, 0, None) == tp.TP_OK
    assert tp.last_error() == ""


def test_training_forward_rejects():
    f = tp.raw.tp_colpar_act_train
    assert f(P[0], P[1], P[2], P[3], None, 4, 64, 256, 4, 0, 0, None) == tp.TP_ERR_NULL
    assert f(P[0], P[1], P[2], P[3], P[3] + 16, 4, 64, 256, 4, 0, 0, None) == tp.TP_ERR_ALIAS
    assert f(P[0], P[1], P[2], P[3], P[4], 4, 64, 256, 4, 0, 5, None) == tp.TP_ERR_UNSUPPORTED
    assert "tp_colpar_act_train" in tp.last_error()


def test_shard_and_group_backward_reject():
    assert tp.raw.tp_mlp_shard_bwd(P[0], P[1], P[2], None, P[4], P[5], P[6], P[7], P[8], P[9], P[10], 4, 64, 256,
                                   4, 0, 0, 0, None) == tp.TP_ERR_NULL
    arr = lambda *xs: tp.partial_array(list(xs))
    U, Y, dU, dX = arr(P[3], P[3] + 4096), arr(P[4], P[4] + 4096), arr(P[6], P[6] + 4096), arr(P[7], P[7] + 8192)
    g = tp.raw.tp_mlp_group_bwd
    assert g(P[0], P[1], P[2], U, Y, P[5], dU, dX, P[8], P[9], P[10], 4, 64, 256, 3, 0, 0, None) == tp.TP_ERR_SHAPE
    assert g(P[0], P[1], None, U, Y, P[5], dU, dX, P[8], P[9], P[10], 4, 64, 256, 2, 0, 0, None) == tp.TP_ERR_NULL
    bad = arr(P[7], P[7])     # two ranks' dX partials on one buffer
    assert g(P[0], P[1], P[2], U, Y, P[5], dU, bad, P[8], P[9], P[10], 4, 64, 256, 2, 0, 0, None) == tp.TP_ERR_ALIAS
    assert g(P[0], P[1], P[2], U, Y, P[5], dU, dX, P[8], P[9], P[10], 0, 64, 256, 2, 0, 0, None) == tp.TP_OK
    assert "" == tp.last_error()


def test_build_compiles_every_kernel_source():
    # every HIP source next to the ABI is part of the library build
    from megatron_tensor_transformer_colpar_amd import build
    hip = sorted(f for f in os.listdir(build.CSRC) if f.endswith(".hip"))
    assert hip and set(hip) <= set(build.SOURCES)
