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
