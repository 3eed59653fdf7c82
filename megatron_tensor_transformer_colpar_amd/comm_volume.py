"""Bytes a real tensor-parallel group moves in its all-reduces: the exchange
that tp_shard_reduce replaces on one GPU.  Reported beside the one-GPU
measurements as the traffic a multi-GPU deployment would add.

"Tensor parallelism" (inference guide), "Walking through a transformer
block" and its worked example: a ring all-reduce of H elements of B bytes
moves about 2 (T - 1) / T * H * B bytes per rank, and a layer runs two of
them (the attention and the MLP residual paths) on the hidden vector of
every token.  Integers throughout; the ring volume is exact whenever T
divides 2 (T - 1) H B, as it does for every shape here.
"""
from __future__ import annotations

from fractions import Fraction


def allreduce_payload_bytes(H: int, elem_bytes: int, tokens: int = 1) -> int:
    """Size of the vector each rank contributes: tokens x H elements."""
    return tokens * H * elem_bytes


def ring_allreduce_bytes_per_rank(H: int, elem_bytes: int, T: int, tokens: int = 1) -> Fraction:
    """Bytes one rank sends (and receives) in a ring all-reduce: a
    reduce-scatter and an all-gather, each T - 1 steps of 1/T of the payload."""
    if T < 1:
        raise ValueError("T must be >= 1")
    return Fraction(2 * (T - 1) * allreduce_payload_bytes(H, elem_bytes, tokens), T)


def stack_ring_bytes_per_rank(layers: int, H: int, elem_bytes: int, T: int, tokens: int = 1,
                              allreduces_per_layer: int = 2) -> Fraction:
    """Ring bytes per rank for one pass of `tokens` tokens through `layers` layers."""
    return layers * allreduces_per_layer * ring_allreduce_bytes_per_rank(H, elem_bytes, T, tokens)
