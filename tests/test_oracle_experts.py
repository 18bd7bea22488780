"""Pins of the oracle's expert computation and combine.

Definitions: glossary "MoE (Mixture of Experts - Mezcla de Expertos)",
section 3 steps 3-4 (SwiGLU experts, weighted sum y = sum_i p_i Expert_i(x)),
section 2 items 2-3 (shared expert always active); "Mixture of experts: por qué
un modelo enorme apenas usa sus parámetros", section "El router ...": compute
per token depends on k, not on the number of experts.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import workloads as W
from tests.dense_ref import dense_forward, f64, swiglu_ffn


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def _run_oracle(inp):
    y, ids, p, margin = oracle.forward(inp)
    return y, ids, p


SWEEP = [
    # T, D, E, k, F, Fs
    (1, 8, 1, 1, 8, 0),
    (3, 16, 2, 1, 32, 0),
    (3, 16, 2, 2, 32, 0),
    (17, 64, 3, 2, 8, 0),
    (17, 64, 8, 3, 256, 0),
    (64, 128, 8, 2, 256, 0),
    (64, 128, 32, 4, 32, 0),
    (33, 64, 32, 8, 32, 0),
    (20, 64, 16, 4, 32, 32),
    (9, 16, 5, 5, 8, 16),
]


@pytest.mark.parametrize("T,D,E,k,F,Fs", SWEEP)
def test_oracle_matches_dense_float64(T, D, E, k, F, Fs):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T * 131 + E)
    y, ids, p = _run_oracle(inp)
    yd, idsd, pd = dense_forward(inp)
    assert np.array_equal(ids, idsd)
    assert np.max(np.abs(p - pd)) < 1e-12
    assert np.max(np.abs(y - yd)) <= 1e-10 * max(_rms(yd), 1e-30)


def test_oracle_matches_dense_on_grid_inputs_with_ties():
    s = W.Shape(T=64, D=16, E=8, k=3, F=16)
    inp = W.make_grid_inputs(s, seed=21)
    y, ids, p = _run_oracle(inp)
    yd, idsd, pd = dense_forward(inp)
    assert np.array_equal(ids, idsd)
    assert np.max(np.abs(y - yd)) <= 1e-10 * _rms(yd)


def test_E1_k1_is_a_dense_swiglu_ffn():
    """One expert, top-1: the layer is exactly a dense SwiGLU FFN (torch float64, F.silu)."""
    s = W.Shape(T=32, D=64, E=1, k=1, F=128)
    inp = W.make_inputs(s, seed=5)
    y, ids, p = _run_oracle(inp)
    assert np.all(ids == 0) and np.all(p == 1.0)
    X = inp.x.double()
    gu = inp.w_gate_up[0].double()
    ref = (torch.nn.functional.silu(X @ gu[:128].T) * (X @ gu[128:].T)) @ inp.w_down[0].double().T
    assert np.max(np.abs(y - ref.numpy())) <= 1e-12 * _rms(ref.numpy())


def test_identical_experts_give_the_ffn_for_any_routing():
    s = W.Shape(T=24, D=32, E=6, k=3, F=16)
    base = W.make_inputs(s, seed=8)
    gu = base.w_gate_up[:1].expand(6, -1, -1).contiguous()
    dn = base.w_down[:1].expand(6, -1, -1).contiguous()
    inp = W.LayerInputs(s, base.x, base.w_g, gu, dn)
    y, ids, p = _run_oracle(inp)
    ref = swiglu_ffn(f64(base.x), f64(base.w_gate_up[0]), f64(base.w_down[0]))
    assert np.max(np.abs(y - ref)) <= 1e-12 * _rms(ref)


def test_k_equals_E_is_a_soft_mixture():
    s = W.Shape(T=16, D=32, E=4, k=4, F=16)
    inp = W.make_inputs(s, seed=6)
    y, ids, p = _run_oracle(inp)
    _, _, _, logits = oracle.route(inp.x, inp.w_g, None, 4)
    gates = sps.softmax(logits.astype(np.float64), axis=1)
    outs = np.stack([swiglu_ffn(f64(inp.x), f64(inp.w_gate_up[e]), f64(inp.w_down[e])) for e in range(4)], 1)
    ref = np.einsum("te,ted->td", gates, outs)
    assert np.max(np.abs(y - ref)) <= 1e-12 * _rms(ref)


def test_relabelling_experts():
    """Permuting the experts (router rows and expert blocks together) leaves y unchanged."""
    s = W.Shape(T=40, D=32, E=8, k=2, F=16)
    inp = W.make_inputs(s, seed=10)
    perm = torch.tensor([3, 7, 0, 5, 1, 6, 2, 4])
    inv = torch.argsort(perm)
    pinp = W.LayerInputs(s, inp.x, inp.w_g[perm].contiguous(), inp.w_gate_up[perm].contiguous(),
                         inp.w_down[perm].contiguous())
    y0, ids0, p0 = _run_oracle(inp)
    y1, ids1, p1 = _run_oracle(pinp)
    # expert e of the original is expert inv[e] of the permuted layer
    assert np.array_equal(np.sort(inv.numpy()[ids0], 1), np.sort(ids1, 1))
    assert np.max(np.abs(y0 - y1)) <= 1e-13 * _rms(y0)


def test_token_independence():
    s = W.Shape(T=50, D=64, E=8, k=2, F=32)
    inp = W.make_inputs(s, seed=12)
    y, _, _ = _run_oracle(inp)
    for t in (0, 17, 49):
        one = W.LayerInputs(s.with_T(1), inp.x[t:t + 1].contiguous(), inp.w_g, inp.w_gate_up, inp.w_down)
        y1, _, _ = _run_oracle(one)
        assert np.array_equal(y1[0], y[t])


def test_scaling_down_projection_by_two_doubles_y_exactly():
    s = W.Shape(T=32, D=64, E=8, k=2, F=32)
    inp = W.make_inputs(s, seed=14)
    y, _, _ = _run_oracle(inp)
    inp2 = W.LayerInputs(s, inp.x, inp.w_g, inp.w_gate_up, (inp.w_down * 2).contiguous())
    y2, _, _ = _run_oracle(inp2)
    assert np.array_equal(y2, 2 * y)


@pytest.mark.parametrize("E", [8, 16, 32, 64])
def test_expert_work_depends_on_k_not_E(E):
    """Multiply-adds of the experts = 3 T k D F for every E (router work aside)."""
    T, D, k, F = 12, 32, 4, 24
    s = W.Shape(T=T, D=D, E=E, k=k, F=F)
    inp = W.make_inputs(s, seed=E)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, None, k)
    y, macs = oracle.experts(inp, ids, p, count_macs=True)
    assert macs == 3 * T * k * D * F


def test_shared_expert_adds_with_weight_one():
    s = W.Shape(T=20, D=32, E=8, k=2, F=16, Fs=24)
    inp = W.make_inputs(s, seed=15)
    y, ids, p = _run_oracle(inp)
    s0 = W.Shape(T=20, D=32, E=8, k=2, F=16)
    y0, ids0, _ = _run_oracle(W.LayerInputs(s0, inp.x, inp.w_g, inp.w_gate_up, inp.w_down))
    ref = swiglu_ffn(f64(inp.x), f64(inp.ws_gate_up), f64(inp.ws_down))
    assert np.array_equal(ids, ids0)
    assert np.max(np.abs((y - y0) - ref)) <= 1e-12 * _rms(ref)
    _, macs = oracle.experts(inp, ids, p, count_macs=True)
    assert macs == 3 * 20 * (2 * 32 * 16 + 32 * 24)


def test_subset_of_tokens_matches_full_run():
    s = W.Shape(T=30, D=32, E=8, k=2, F=16)
    inp = W.make_inputs(s, seed=16)
    y, ids, p = _run_oracle(inp)
    tok = np.array([29, 3, 3, 0])
    ys = oracle.experts(inp, ids, p, tokens=tok)
    assert np.array_equal(ys, y[tok])


def test_hand_worked_closed_form():
    """A two-dimensional layer small enough to evaluate by hand.

    D=2, E=3, k=2, F=1, x = (1, 0).  Router rows (1,0), (0,0), (-1,0) give logits
    (1, 0, -1): experts 0 and 1 are chosen with p = (e/(e+1), 1/(e+1)).
    Expert e has gate row (a_e, 0), up row (b_e, 0), down column (c_e, d_e), so
    its output is SiLU(a_e) * b_e * (c_e, d_e) with SiLU(a) = a / (1 + e^-a).
    """
    a = [1.0, 2.0, 0.5]
    b = [2.0, -1.0, 4.0]
    c = [0.5, 1.0, 8.0]
    d = [-1.0, 0.25, 2.0]
    s = W.Shape(T=1, D=2, E=3, k=2, F=1)
    bf = torch.bfloat16
    x = torch.tensor([[1.0, 0.0]], dtype=bf)
    w_g = torch.tensor([[1.0, 0.0], [0.0, 0.0], [-1.0, 0.0]], dtype=bf)
    w_gu = torch.tensor([[[a[e], 0.0], [b[e], 0.0]] for e in range(3)], dtype=bf)
    w_dn = torch.tensor([[[c[e]], [d[e]]] for e in range(3)], dtype=bf)
    y, ids, p = _run_oracle(W.LayerInputs(s, x, w_g, w_gu, w_dn))
    e_ = math.e
    p0, p1 = e_ / (e_ + 1.0), 1.0 / (e_ + 1.0)
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    silu2 = 2.0 / (1.0 + math.exp(-2.0))
    expect = [p0 * silu1 * 2.0 * 0.5 + p1 * silu2 * -1.0 * 1.0,
              p0 * silu1 * 2.0 * -1.0 + p1 * silu2 * -1.0 * 0.25]
    assert ids.tolist() == [[0, 1]]
    assert abs(p[0, 0] - p0) < 1e-15 and abs(p[0, 1] - p1) < 1e-15
    assert np.max(np.abs(y[0] - np.array(expect))) < 1e-14
