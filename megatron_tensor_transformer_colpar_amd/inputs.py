"""Seeded synthetic inputs, shared by the parity tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage precision
(fp32, then bf16 round-to-nearest-even).  It holds none of the block's
arithmetic, so both the HIP path and the oracle can consume what it makes.

Generator: numpy ``PCG64`` seeded with ``SeedSequence([seed, workload, layer,
tensor, shard])``; values are ``std * standard_normal`` in fp64, rounded to fp32
and, for bf16 tensors, to bf16 (RNE, quiet NaNs kept).  ``N(0, s)`` means
standard deviation ``s``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# tensor ids for the seed sequence
X_ID, W1_ID, B1_ID, W2_ID, CTX_ID, WO_ID = 0, 1, 2, 3, 4, 5
WG_ID, WU_ID, BG_ID, BU_ID = 6, 7, 8, 9   # gated first layer: gate and up weights and biases
WQ_ID, WK_ID, WV_ID, BQ_ID, BK_ID, BV_ID = 10, 11, 12, 13, 14, 15   # attention projections
Q_ID, K_ID, V_ID, LEN_ID = 16, 17, 18, 19                            # attention core operands
HEAD_DIM = 128


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaNs stay quiet NaNs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Synth:
    """A host tensor in its storage precision.

    ``dtype`` is "bf16" or "f32".  ``data`` holds the storage array (uint16 bf16
    bit patterns, or float32).  ``f64`` gives the exact values as float64.
    """

    dtype: str
    data: np.ndarray

    @property
    def shape(self):
        return self.data.shape

    @property
    def f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.data) if self.dtype == "bf16" else self.data

    @property
    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def transposed(self) -> "Synth":
        """A contiguous copy of the transpose (2-D), same precision."""
        return Synth(self.dtype, np.ascontiguousarray(self.data.T))

    def rows(self, idx) -> "Synth":
        return Synth(self.dtype, np.ascontiguousarray(self.data[idx]))

    def torch(self, device="cuda"):
        """Upload to a torch tensor (bf16 or fp32) on ``device``."""
        import torch

        if self.dtype == "bf16":
            t = torch.from_numpy(self.data.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.data)
        return t.to(device)


def from_values(values, dtype: str) -> Synth:
    """Round fp64/fp32 values to the storage precision."""
    v32 = np.asarray(values, dtype=np.float32)
    if dtype == "bf16":
        return Synth("bf16", f32_to_bf16_bits(v32))
    if dtype == "f32":
        return Synth("f32", np.ascontiguousarray(v32))
    raise ValueError("dtype must be 'bf16' or 'f32'")


def normal(shape, std: float, dtype: str, *, seed: int = 0, workload: int = 0,
           layer: int = 0, tensor: int = 0, shard: int = 0) -> Synth:
    """``std * N(0,1)`` of the given shape, rounded to ``dtype``.  std == 0 gives zeros."""
    ss = np.random.SeedSequence([seed, workload, layer, tensor, shard])
    rng = np.random.Generator(np.random.PCG64(ss))
    if std == 0:
        return from_values(np.zeros(shape), dtype)
    return from_values(std * rng.standard_normal(shape), dtype)


def row_sample(M: int, n: int, *, seed: int = 0, include_ends: bool = True) -> np.ndarray:
    """A seeded, sorted subset of ``n`` token rows of ``M`` (always first and last)."""
    if n >= M:
        return np.arange(M)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 991, M, n])))
    pick = set(rng.choice(M, size=n, replace=False).tolist())
    if include_ends:
        pick |= {0, M - 1}
    return np.array(sorted(pick), dtype=np.int64)


# ---------------------------------------------------------------------------
# Workloads: the shapes and value distributions of the block's standard cases.
# M tokens, hidden H, FFN width F, TP degree T; attention width A = heads * 128.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str
    M: int
    H: int
    F: int
    T: int
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.01
    A: int = 0          # attention width (heads * head_dim); 0 = no out-projection
    layers: int = 1


WORKLOADS = {
    "tiny_f32": Workload(1, "tiny_f32", "f32", M=8, H=256, F=1024, T=2, b_std=0.0),
    "gpt_block_shard": Workload(2, "gpt_block_shard", "bf16", M=2048, H=4096, F=16384, T=4),
    "decode": Workload(3, "decode", "bf16", M=32, H=8192, F=32768, T=8, A=8192),
    "prefill": Workload(4, "prefill", "bf16", M=8192, H=8192, F=32768, T=8),
    "stack80": Workload(5, "stack80", "bf16", M=8, H=8192, F=32768, T=8, A=8192, layers=80),
}


def gated_inputs(w: Workload, *, M: int | None = None, seed: int = 0, layer: int = 0,
                 shard_only: int | None = None):
    """X [M,H], Wg [H,F], Wu [H,F], bg [F], bu [F] for the gated first layer,
    drawn like the plain layer's X, W1 and b1 (same distributions)."""
    M = w.M if M is None else M
    kw = dict(seed=seed, workload=w.wid, layer=layer)
    X = normal((M, w.H), w.x_std, w.dtype, tensor=X_ID, **kw)
    if shard_only is None:
        F, sh = w.F, 0
    else:
        F, sh = w.F // w.T, shard_only + 1
    Wg = normal((w.H, F), w.w_std, w.dtype, tensor=WG_ID, shard=sh, **kw)
    Wu = normal((w.H, F), w.w_std, w.dtype, tensor=WU_ID, shard=sh, **kw)
    bg = normal((F,), w.b_std, w.dtype, tensor=BG_ID, shard=sh, **kw)
    bu = normal((F,), w.b_std, w.dtype, tensor=BU_ID, shard=sh, **kw)
    return X, Wg, Wu, bg, bu


def mlp_inputs(w: Workload, *, M: int | None = None, seed: int = 0, layer: int = 0,
               shard_only: int | None = None):
    """X [M,H], W1 [H,F], b1 [F], W2 [F,H] as Synth (logical [in, out] weights).

    With ``shard_only=i`` only rank i's blocks are drawn, as stand-alone
    matrices W1_i [H, F/T], b1_i [F/T], W2_i [F/T, H] (seeded per shard).
    """
    M = w.M if M is None else M
    kw = dict(seed=seed, workload=w.wid, layer=layer)
    X = normal((M, w.H), w.x_std, w.dtype, tensor=X_ID, **kw)
    if shard_only is None:
        F, sh = w.F, 0
    else:
        F, sh = w.F // w.T, shard_only + 1
    W1 = normal((w.H, F), w.w_std, w.dtype, tensor=W1_ID, shard=sh, **kw)
    b1 = normal((F,), w.b_std, w.dtype, tensor=B1_ID, shard=sh, **kw)
    W2 = normal((F, w.H), w.w_std, w.dtype, tensor=W2_ID, shard=sh, **kw)
    return X, W1, b1, W2


def outproj_inputs(w: Workload, *, M: int | None = None, seed: int = 0, layer: int = 0,
                   shard: int = 0):
    """Rank ``shard``'s attention context ctx_i [M, A/T] and its W_o row block [A/T, H]."""
    M = w.M if M is None else M
    As = w.A // w.T
    kw = dict(seed=seed, workload=w.wid, layer=layer, shard=shard + 1)
    ctx = normal((M, As), 1.0, w.dtype, tensor=CTX_ID, **kw)
    Wo = normal((As, w.H), w.w_std, w.dtype, tensor=WO_ID, **kw)
    return ctx, Wo


# ---------------------------------------------------------------------------
# Attention front half: rank i's heads.  Sequences of a prefill batch are
# consecutive token rows (row b*S + s); a decode step is one query per
# sequence against a cache of Lk positions.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnShape:
    wid: int
    name: str
    Bs: int        # sequences
    Sq: int        # queries per sequence
    Lk: int        # keys per sequence (cache capacity)
    nh: int        # query heads of the rank
    nkv: int       # key/value heads of the rank
    H: int         # hidden size (projection input)
    T: int         # TP degree (the full model has T * nh heads)
    causal: bool = True


ATTN_SHAPES = {
    # the 8192-token prefill (4 sequences of 2048), 64 heads of 128 over 8 ranks
    "prefill": AttnShape(6, "prefill", Bs=4, Sq=2048, Lk=2048, nh=8, nkv=8, H=8192, T=8),
    # the 2048-token GPT-style block, 32 heads of 128 over 4 ranks
    "gpt_block_shard": AttnShape(7, "gpt_block_shard", Bs=1, Sq=2048, Lk=2048, nh=8, nkv=8, H=4096, T=4),
    # decode: one new token per sequence against 2048 cached positions
    "decode": AttnShape(8, "decode", Bs=32, Sq=1, Lk=2048, nh=8, nkv=8, H=8192, T=8),
}


def attn_core_inputs(Bs: int, Sq: int, Lk: int, nh: int, nkv: int, *, seed: int = 0, wid: int = 0,
                     q_std: float = 1.0, k_std: float = 1.0, v_std: float = 1.0):
    """Q [Bs, Sq, nh*128], K and V [Bs, Lk, nkv*128], bf16, N(0, std) each."""
    kw = dict(seed=seed, workload=wid)
    Q = normal((Bs, Sq, nh * HEAD_DIM), q_std, "bf16", tensor=Q_ID, **kw)
    K = normal((Bs, Lk, nkv * HEAD_DIM), k_std, "bf16", tensor=K_ID, **kw)
    V = normal((Bs, Lk, nkv * HEAD_DIM), v_std, "bf16", tensor=V_ID, **kw)
    return Q, K, V


def ragged_lengths(Bs: int, lo: int, hi: int, *, seed: int = 0) -> np.ndarray:
    """Seeded cache lengths in [lo, hi] (int32), the first and last pinned to hi and lo."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, LEN_ID, Bs, lo, hi])))
    n = rng.integers(lo, hi + 1, size=Bs).astype(np.int32)
    if Bs > 0:
        n[0] = hi
    if Bs > 1:
        n[-1] = lo
    return n


def qkv_inputs(H: int, A: int, Akv: int, T: int, *, M: int, dtype: str = "bf16", seed: int = 0, wid: int = 0,
               x_std: float = 1.0, w_std: float = 0.02, b_std: float = 0.01, shard_only: int | None = None):
    """X [M,H], Wq [H,A], Wk [H,Akv], Wv [H,Akv], bq [A], bk [Akv], bv [Akv] (logical
    [in, out] weights).  With ``shard_only=i`` only rank i's column blocks are
    drawn, as stand-alone [H, A/T] / [H, Akv/T] matrices."""
    kw = dict(seed=seed, workload=wid)
    X = normal((M, H), x_std, dtype, tensor=X_ID, **kw)
    if shard_only is None:
        a, akv, sh = A, Akv, 0
    else:
        a, akv, sh = A // T, Akv // T, shard_only + 1
    Wq = normal((H, a), w_std, dtype, tensor=WQ_ID, shard=sh, **kw)
    Wk = normal((H, akv), w_std, dtype, tensor=WK_ID, shard=sh, **kw)
    Wv = normal((H, akv), w_std, dtype, tensor=WV_ID, shard=sh, **kw)
    bq = normal((a,), b_std, dtype, tensor=BQ_ID, shard=sh, **kw)
    bk = normal((akv,), b_std, dtype, tensor=BK_ID, shard=sh, **kw)
    bv = normal((akv,), b_std, dtype, tensor=BV_ID, shard=sh, **kw)
    return X, Wq, Wk, Wv, bq, bk, bv
