"""What the C ABI enqueues, read from the launch-recording CPU build (runs
only inside the host sanitizer run; skipped elsewhere).

The layer driver's schedule is fixed by "Tensor parallelism" (inference
guide), "Walking through a transformer block": two all-reduces per layer,
one on the attention residual path after the head-sharded out-projection,
one on the MLP residual path after the row-parallel down-projection; and by
"Slice the matrix itself", "All-Reduce Synchronization": the column-parallel
up-projection needs no exchange before the row-parallel one."""
import ctypes

import pytest

from tests.host_double import plugin

pytestmark = pytest.mark.skipif(not plugin.ACTIVE, reason="runs inside the host sanitizer run only")

GEMM, GEMV, GEMM_F32, ATTN, COLSUM, REDUCE = range(6)
EPI_BIAS_GELU, EPI_STORE_F32 = 0, 1
# fake device addresses, 64 GiB apart: the recorder never dereferences them
P = [(k + 1) << 36 for k in range(40)]


def arr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def run_layer(M, H=8192, F=32768, A=8192, T=8):
    from megatron_tensor_transformer_colpar_amd import tp

    plugin.recorder.rec_reset()
    ctx, Y, parts = arr(P[10:10 + T]), arr(P[20:20 + T]), arr(P[30:30 + T])
    st = tp.raw.tp_layer_fwd(P[0], P[1], ctx, P[2], A, P[3], P[4], P[5], Y, parts, M, H, F, T, None)
    assert st == tp.TP_OK, tp.last_error()
    return plugin.log()


@pytest.mark.parametrize("M", [8, 4096])
def test_layer_runs_exactly_two_reductions(M):
    H, F, A, T = 8192, 32768, 8192, 8
    log = run_layer(M, H, F, A, T)
    kinds = [e[0] for e in log]
    assert kinds.count(REDUCE) == 2
    proj = GEMV if M <= 32 else GEMM
    assert kinds == [proj, REDUCE, proj, proj, REDUCE]
    oproj, red1, up, down, red2 = log
    # every rank's head-sharded out-projection partial, K = A/T, in one launch
    assert (oproj[1], oproj[2], oproj[3], oproj[4], oproj[5]) == (EPI_STORE_F32, M, H, A // T, T)
    # first reduce: residual in, bf16 row-RMS copy out
    assert red1[1] == 3 and red1[5] == T and red1[6] == 1 and red1[2:4] == (M, H)
    # the column-parallel up-projection with bias + GeLU: no exchange before it
    assert (up[1], up[2], up[3], up[4], up[5]) == (EPI_BIAS_GELU, M, F // T, H, T)
    # the row-parallel down-projection's fp32 partials, then the second reduce into h
    assert (down[1], down[2], down[3], down[4], down[5]) == (EPI_STORE_F32, M, H, F // T, T)
    assert red2[1] == 1 and red2[5] == T and red2[6] == 0
    assert plugin.recorder.rec_violations() == 0


def test_mlp_shard_is_two_launches_and_empty_calls_none():
    from megatron_tensor_transformer_colpar_amd import tp

    plugin.recorder.rec_reset()
    assert tp.raw.tp_mlp_shard_fwd(P[0], P[1], P[2], P[3], P[4], P[5], 8192, 8192, 32768, 8, 3, 0, None) == 0
    log = plugin.log()
    assert [e[0] for e in log] == [GEMM, GEMM]
    assert (log[0][1], log[0][3], log[0][4]) == (EPI_BIAS_GELU, 4096, 8192)
    assert (log[1][1], log[1][3], log[1][4]) == (EPI_STORE_F32, 8192, 4096)
    plugin.recorder.rec_reset()
    assert tp.raw.tp_mlp_shard_fwd(P[0], P[1], P[2], P[3], P[4], P[5], 0, 8192, 32768, 8, 3, 0, None) == 0
    assert tp.raw.tp_layer_fwd(P[0], P[1], arr(P[10:18]), P[2], 8192, P[3], P[4], P[5], arr(P[20:28]),
                               arr(P[30:38]), 0, 8192, 32768, 8, None) == 0
    assert plugin.log() == []


@pytest.mark.parametrize("M,kind", [(1, GEMV), (32, GEMV), (33, GEMM)])
def test_decode_path_below_33_tokens(M, kind):
    from megatron_tensor_transformer_colpar_amd import tp

    plugin.recorder.rec_reset()
    assert tp.raw.tp_colpar_gelu(P[0], P[1], P[2], P[3], M, 8192, 32768, 8, 0, 0, None) == 0
    assert tp.raw.tp_colpar_gelu(P[0], P[1], P[2], P[3], M, 256, 1024, 2, 1, 1, None) == 0
    assert [e[0] for e in plugin.log()] == [kind, GEMM_F32]


def test_noalloc_shard_stages_in_the_library_buffer():
    # the no-allocation variant runs the same two launches as tp_mlp_shard_fwd,
    # with Y_i in the library's staging buffer; at the limit it still launches
    from megatron_tensor_transformer_colpar_amd import tp

    plugin.recorder.rec_reset()
    assert tp.raw.tp_mlp_shard_fwd_noalloc(P[0], P[1], P[2], P[3], P[5], 8, 8192, 32768, 8, 3, 0, None) == 0
    assert tp.raw.tp_mlp_shard_fwd_noalloc(P[0], P[1], P[2], P[3], P[5], 2048, 4096, 4096, 1, 0, 0, None) == 0
    log = plugin.log()
    assert [e[0] for e in log] == [GEMV, GEMV, GEMM, GEMM]
    assert [e[1] for e in log] == [EPI_BIAS_GELU, EPI_STORE_F32] * 2
    assert plugin.recorder.rec_violations() == 0
