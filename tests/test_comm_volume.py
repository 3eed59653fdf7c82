"""The all-reduce volume helper against the worked example of "Tensor
parallelism" (inference guide), "Walking through a transformer block":
H = 8192, bf16 (B = 2), T = 8, one residual all-reduce has a 16 KiB payload
per rank and a ring volume of about 28 KiB per rank; two collectives per
layer over 80 layers come to about 4.4 MB per token per decode step."""
import json
import os
from fractions import Fraction

from megatron_tensor_transformer_colpar_amd import comm_volume as cv

KiB, MiB = 1024, 1024 * 1024
# the example's figures, with their citation, in tests/golden/
EX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ring_allreduce_worked_example.json")))


def test_payload_of_the_worked_example():
    assert cv.allreduce_payload_bytes(EX["hidden"], EX["bytes_per_element"]) == EX["payload_bytes_per_rank"]


def test_ring_volume_of_the_worked_example():
    v = cv.ring_allreduce_bytes_per_rank(EX["hidden"], EX["bytes_per_element"], EX["tp"])
    assert v == EX["ring_bytes_per_rank_approx"]   # 2 * 7/8 * 16 KiB, exactly 28 KiB
    assert v.denominator == 1


def test_eighty_layer_decode_step():
    v = cv.stack_ring_bytes_per_rank(EX["layers"], EX["hidden"], EX["bytes_per_element"], EX["tp"])
    assert v == EX["layers"] * EX["allreduces_per_layer"] * EX["ring_bytes_per_rank_approx"] == 4480 * KiB
    assert abs(float(v) / MiB - EX["decode_step_megabytes_approx"]) < 0.05   # the page rounds to one decimal


def test_degenerate_and_two_rank_groups():
    # one rank exchanges nothing; two ranks each send exactly the payload
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 1) == 0
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 2) == 16 * KiB
    # tokens scale the payload linearly (decode M = 8: 8 token vectors)
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 8, tokens=8) == 8 * 28 * KiB
    # the volume tends to twice the payload as T grows
    assert cv.ring_allreduce_bytes_per_rank(8192, 2, 1024) == Fraction(2 * 1023 * 16 * KiB, 1024)
