"""The all-reduce volume helper against the worked example of "Tensor
parallelism" (inference guide), "Walking through a transformer block":
H = 8192, bf16 (B = 2), T = 8, one residual all-reduce has a 16 KiB payload
per rank and a ring volume of about 28 KiB per rank; two collectives per
layer over 80 layers come to about 4.4 MB per token per decode step."""
from fractions import Fraction

from megatron_tensor_transformer_colpar_amd import comm_volume as cv

KiB, MiB = 1024, 1024 * 1024


def test_payload_of_the_worked_example():
    assert cv.allreduce_payload_bytes(8192, 2) == 16 * KiB


def test_ring_volume_of_the_worked_example():
    v = cv.ring_allreduce_bytes_per_rank(8192, 2, 8)
    assert v == 28 * KiB                     # 2 * 7/8 * 16 KiB, exactly
    assert v.denominator == 1


def test_eighty_layer_decode_step():
    v = cv.stack_ring_bytes_per_rank(80, 8192, 2, 8)
    assert v == 80 * 2 * 28 * KiB == 4480 * KiB
    assert abs(float(v) / MiB - 4.4) < 0.05  # the page's "about 4.4 MB"


def test_degenerate_and_two_rank_groups():
    # one rank exchanges nothing; two ranks each send exactly the payload
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 1) == 0
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 2) == 16 * KiB
    # tokens scale the payload linearly (decode M = 8: 8 token vectors)
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 8, tokens=8) == 8 * 28 * KiB
    # the volume tends to twice the payload as T grows
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 1024) == Fraction(2 * 1023 * 16 * KiB, 1024)
