"""Seeded input generator: determinism, recipe and bf16 rounding.  CPU only."""
import numpy as np
import pytest
import torch

from nystr_linear_attention_amd import workloads as wl


def test_five_workloads_shapes():
    shapes = [(w.heads, w.N, w.d, w.m) for w in wl.WORKLOADS]
    assert shapes == [(1, 196, 32, 49), (8, 3136, 64, 49), (160, 784, 64, 49),
                      (2, 16384, 64, 64), (32, 3136, 64, 49)]
    assert wl.HEADLINE.name == "lap_f32_pvt1_b8_n3136_d64_m49"
    assert [w.seed for w in wl.WORKLOADS] == [1000, 1001, 1002, 1003, 1004]


def test_deterministic_and_ordered():
    w = wl.small_case(4, 4, 8, 2, 2, B=2, H=1, seed=5)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for key in "qkv":
        assert np.array_equal(a[key], b[key])
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 1, 16, 8)).astype(np.float32)
    k = rng.standard_normal((2, 1, 16, 8)).astype(np.float32)
    assert np.array_equal(a["q"], q) and np.array_equal(a["k"], k)


def test_shared_qk_is_same_array():
    w = wl.WORKLOADS[4].replace(B=1, H=1)
    x = wl.make_inputs(w)
    assert x["k"] is x["q"]


def test_headline_scale():
    w = wl.HEADLINE.replace(B=2)
    x = wl.make_inputs(w)
    # N(0,1)/sqrt(64)*4 -> standard deviation 0.5 for Q, K and V
    for key in "qkv":
        assert abs(float(np.std(x[key])) - 0.5) < 0.01


@pytest.mark.parametrize("seed", [0, 1])
def test_bf16_rne_matches_torch(seed):
    r = np.random.default_rng(seed)
    x = np.concatenate([r.standard_normal(20000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -0.0, 65504.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
