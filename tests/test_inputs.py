"""The seeded input generator: host bf16 rounding against torch's (round to
nearest even) bit for bit, determinism of the seeds, and the workload shapes."""
import numpy as np
import pytest
import torch

from megatron_tensor_transformer_colpar_amd import inputs


def torch_bits(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    assert np.array_equal(inputs.f32_to_bf16_bits(x), torch_bits(x))


def test_bf16_rne_ties_subnormals_and_specials():
    # exact ties between two bf16 neighbours go to the even one
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x00008000, 0x00018000, 0x7F7F8000],
                    dtype=np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38, -3.4e38], dtype=np.float32)
    x = np.concatenate([ties, special])
    assert np.array_equal(inputs.f32_to_bf16_bits(x), torch_bits(x))
    got = inputs.f32_to_bf16_bits(np.array([0x3F808000, 0x3F818000], dtype=np.uint32).view(np.float32))
    assert got.tolist() == [0x3F80, 0x3F82]
    nan = inputs.f32_to_bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    back = inputs.bf16_bits_to_f32(nan)
    assert np.isnan(back).all() and ((nan & 0x0040) != 0).all()


def test_roundtrip_is_exact_for_bf16_values():
    s = inputs.normal((64, 64), 0.02, "bf16", tensor=1)
    again = inputs.from_values(s.f64, "bf16")
    assert np.array_equal(s.data, again.data)


def test_seeds_are_deterministic_and_distinct():
    a = inputs.normal((8, 8), 1.0, "f32", workload=2, tensor=1)
    b = inputs.normal((8, 8), 1.0, "f32", workload=2, tensor=1)
    c = inputs.normal((8, 8), 1.0, "f32", workload=2, tensor=3)
    assert np.array_equal(a.data, b.data) and not np.array_equal(a.data, c.data)


def test_distribution_is_standard_deviation():
    s = inputs.normal((512, 512), 0.02, "f32", tensor=5)
    assert abs(s.f64.std() - 0.02) < 0.0005 and abs(s.f64.mean()) < 0.0005


def test_workload_shapes():
    w = inputs.WORKLOADS["gpt_block_shard"]
    X, W1, b1, W2 = inputs.mlp_inputs(w, M=16)
    assert X.shape == (16, 4096) and W1.shape == (4096, 16384) and b1.shape == (16384,)
    assert W2.shape == (16384, 4096) and X.dtype == "bf16"
    t = inputs.WORKLOADS["tiny_f32"]
    X, W1, b1, W2 = inputs.mlp_inputs(t)
    assert X.dtype == "f32" and not b1.f64.any()
    d = inputs.WORKLOADS["decode"]
    ctx, Wo = inputs.outproj_inputs(d, M=8, shard=3)
    assert ctx.shape == (8, 1024) and Wo.shape == (1024, 8192)


def test_row_sample_keeps_ends():
    r = inputs.row_sample(2048, 16)
    assert r[0] == 0 and r[-1] == 2047 and len(set(r.tolist())) == len(r) and np.all(np.diff(r) > 0)
