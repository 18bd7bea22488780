"""Checks of the seeded input generator and the size arithmetic (no layer math)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")
M64 = (1 << 64) - 1


def _mix(z):
    """SplitMix64 output function, written from its published definition."""
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _py_normal(seed, tag, i, std):
    key = _mix(_mix(seed) ^ tag)
    w = _mix((key + ((i // 2) + 1) * 0x9E3779B97F4A7C15) & M64)
    u1 = ((w >> 32) + 0.5) / 2.0 ** 32
    u2 = ((w & 0xFFFFFFFF) + 0.5) / 2.0 ** 32
    r = math.sqrt(-2.0 * math.log(u1))
    z = r * (math.cos(2 * math.pi * u2) if i % 2 == 0 else math.sin(2 * math.pi * u2))
    return float(np.float32(z * std))


def test_generator_follows_its_definition():
    got = W.normal_f32((101,), seed=0, tag=W.TAG_X, std=1.0, start=7).numpy()
    ref = [_py_normal(0, W.TAG_X, 7 + j, 1.0) for j in range(101)]
    assert np.max(np.abs(got - np.array(ref, np.float32))) <= 2e-7 * np.max(np.abs(ref))
    b = W.normal_bf16((101,), seed=0, tag=W.TAG_X, std=1.0, start=7)
    assert torch.equal(b, torch.from_numpy(got).to(torch.bfloat16))


def test_generator_statistics_and_determinism():
    a = W.normal_bf16((1 << 20,), seed=1, tag=W.TAG_W_DOWN, std=0.02)
    b = W.normal_bf16((1 << 20,), seed=1, tag=W.TAG_W_DOWN, std=0.02)
    assert torch.equal(a, b)
    f = a.double().numpy()
    assert abs(f.mean()) < 1e-4 and abs(f.std() - 0.02) < 1e-4
    kurt = np.mean((f / f.std()) ** 4)
    assert abs(kurt - 3.0) < 0.05  # normal tails, not clipped
    c = W.normal_bf16((1 << 20,), seed=2, tag=W.TAG_W_DOWN, std=0.02)
    assert not torch.equal(a, c)


def test_x_is_prefix_consistent_and_weights_do_not_depend_on_T():
    s = W.WORKLOADS["tiny"].shape
    i64 = W.make_inputs(s.with_T(64))
    i8 = W.make_inputs(s.with_T(8))
    assert torch.equal(i64.x[:8], i8.x)
    assert torch.equal(i64.w_gate_up, i8.w_gate_up) and torch.equal(i64.w_g, i8.w_g)


def test_skew_bias_closed_form():
    b = W.skew_bias(8).double().numpy()
    ref = [3.0 * math.log(1.0 / (e + 1) ** 1.2) for e in range(8)]
    assert np.max(np.abs(b - ref)) < 1e-6
    assert abs(b[1] - (-2.4953)) < 1e-4 and abs(b[7] - (-7.4860)) < 1e-4


def test_grid_inputs_are_exact_eighths():
    g = W.grid_bf16((4096,), 0, 1).double().numpy()
    assert np.all(g * 8 == np.round(g * 8)) and g.min() >= -2 and g.max() <= 2


def test_workload_shapes_match_the_pages():
    pages = json.load(open(GOLDEN))
    m = W.WORKLOADS["mixtral_prefill"].shape
    assert (m.E, m.k) == (pages["coarse_mixtral_8x7b"]["num_experts"], pages["coarse_mixtral_8x7b"]["experts_per_token"])
    d = W.WORKLOADS["deepseek_fine"].shape
    assert (d.E, d.k) == (pages["fine_deepseek_v3"]["num_experts"], pages["fine_deepseek_v3"]["experts_per_token"])
    assert d.Fs > 0
    g = W.WORKLOADS["gptoss_decode"].shape
    assert (g.E, g.k) == (pages["gpt_oss_20b"]["num_experts"], pages["gpt_oss_20b"]["experts_per_token"])


def test_active_parameter_arithmetic_of_the_pages():
    """gpt-oss-20b: 21B total, 4 of 32 experts, ~3.6B active, bf16 at ~800 GB/s -> ~111 tok/s."""
    pg = json.load(open(GOLDEN))["gpt_oss_20b"]
    est = pg["bandwidth_bytes_per_s"] / (pg["active_params"] * pg["bytes_per_param"])
    assert round(est) == pg["estimated_tokens_per_s"]
    s = W.WORKLOADS["gptoss_decode"].shape
    # routed active / routed total = k / E exactly
    routed_active = W.active_params(s) - s.D * s.E
    assert routed_active * s.E == (W.total_params(s) - s.D * s.E) * s.k
    assert W.active_params(s) == 99_624_960 and W.total_params(s) == 796_354_560
    # 21B = other + R, 3.6B = other + R k/E  ->  R = routed expert params of the model
    R = (pg["total_params"] - pg["active_params"]) / (1 - pg["experts_per_token"] / pg["num_experts"])
    layers = R / (s.E * W.expert_params(s))
    assert 24 <= layers <= 26


def test_flop_and_byte_counts():
    s = W.WORKLOADS["mixtral_prefill"].shape
    assert W.algorithmic_flops(s) == 2 * 4096 * 4096 * 8 + 6 * 4096 * 2 * 4096 * 14336
    assert abs(W.algorithmic_flops(s) / 1e12 - 2.8865) < 1e-3
    assert W.gate_up_flops(s) + W.down_flops(s) + 2 * s.T * s.D * s.E == W.algorithmic_flops(s)
    c = W.WORKLOADS["gptoss_decode"].shape
    assert abs(W.algorithmic_bytes(c, 32) / 1e9 - 1.594) < 2e-3
