"""Test-side glue: upload seeded inputs in the library's layout, run the shard
through the C ABI, and compare with the oracle.  Tolerances (relative
Frobenius norm of the difference): 5e-3 for bf16 storage with fp32
accumulation, 1e-5 for fp32."""
from __future__ import annotations

import numpy as np
import torch

from megatron_tensor_transformer_colpar_amd import inputs

TOL = {"bf16": 5e-3, "f32": 1e-5}


def rel_fro(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def torch_dtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def tp_dtype(dt: str) -> int:
    from megatron_tensor_transformer_colpar_amd import tp

    return tp.TP_BF16 if dt == "bf16" else tp.TP_F32


class DeviceMLP:
    """X, W1^T, b1, W2^T on the GPU (weights stored K-contiguous)."""

    def __init__(self, X, W1, b1, W2, device="cuda"):
        self.dt = X.dtype
        self.M, self.H = X.shape
        self.F = W1.shape[1]
        self.X = X.torch(device)
        self.W1t = W1.transposed().torch(device)
        self.b1 = None if b1 is None else b1.torch(device)
        self.W2t = W2.transposed().torch(device)

    def shard(self, T, i, use_fused=True):
        """Run rank i's share; returns (Y_i, Z_i) device tensors."""
        from megatron_tensor_transformer_colpar_amd import tp

        Fs = self.F // T
        Y = torch.empty(self.M, Fs, dtype=torch_dtype(self.dt), device=self.X.device)
        Z = torch.empty(self.M, self.H, dtype=torch.float32, device=self.X.device)
        dt = tp_dtype(self.dt)
        if use_fused:
            tp.tp_mlp_shard_fwd(self.X, self.W1t, self.b1, self.W2t, Y, Z, self.M, self.H, self.F, T, i, dt)
        else:
            tp.tp_colpar_gelu(self.X, self.W1t, self.b1, Y, self.M, self.H, self.F, T, i, dt)
            tp.tp_rowpar_partial(Y, self.W2t, Z, self.M, self.H, self.F, T, i, dt)
        return Y, Z

    def all_shards_reduced(self, T, use_fused=True):
        from megatron_tensor_transformer_colpar_amd import tp

        parts = [self.shard(T, i, use_fused) for i in range(T)]
        Z = torch.empty(self.M, self.H, dtype=torch.float32, device=self.X.device)
        tp.tp_shard_reduce([p[1] for p in parts], T, None, Z, None, self.M, self.H)
        return parts, Z
