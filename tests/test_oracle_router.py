"""Pins of the oracle's router: logits, top-k selection and the softmax over the chosen.

The router is defined by "Mixture of experts: por qué un modelo enorme apenas
usa sus parámetros", section "El router: la pieza que de verdad decide", and
by the glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 2
diagram row 2: p = Softmax(TopK(W_g x)).
"""
import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import workloads as W


def _grid(T, D, E, k, seed=3, bias=False):
    return W.make_grid_inputs(W.Shape(T=T, D=D, E=E, k=k, F=8, router_bias=bias), seed=seed)


@pytest.mark.parametrize("T,D,E,k", [(64, 128, 8, 2), (33, 64, 32, 4), (17, 256, 256, 8), (5, 8, 3, 3)])
def test_logits_exact_on_grid_inputs(T, D, E, k):
    """Grid inputs (multiples of 1/8) make every logit an exact fp32 value:
    integer arithmetic gives it with no rounding at all."""
    inp = _grid(T, D, E, k)
    _, _, _, logits = oracle.route(inp.x, inp.w_g, None, k)
    xi = (inp.x.to(torch.float64).numpy() * 8).astype(np.int64)
    wi = (inp.w_g.to(torch.float64).numpy() * 8).astype(np.int64)
    exact = (xi @ wi.T).astype(np.float64) / 64.0
    assert np.array_equal(logits.astype(np.float64), exact)


def test_logits_within_inner_product_bound():
    """Random inputs: the fp32 logit is within one fp32 rounding of the exact
    float64 inner product (the oracle accumulates in double, rounds once)."""
    s = W.Shape(T=40, D=2880, E=32, k=4, F=8)
    inp = W.make_inputs(s, seed=11)
    _, _, _, logits = oracle.route(inp.x, inp.w_g, None, s.k)
    X = inp.x.to(torch.float64).numpy()
    G = inp.w_g.to(torch.float64).numpy()
    exact = X @ G.T
    # |fp32(s) - s| <= 2^-24 |s| plus the double accumulation error (D * 2^-53 * sum|x w|)
    bound = np.abs(exact) * 2.0 ** -24 + s.D * 2.0 ** -53 * (np.abs(X) @ np.abs(G).T) * 1.01
    assert np.all(np.abs(logits.astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("T,D,E,k", [(64, 128, 8, 2), (50, 64, 32, 4), (20, 32, 256, 8), (9, 16, 5, 5)])
def test_topk_matches_stable_argsort(T, D, E, k):
    """Ids = first k of a stable descending sort of the fp32 logits (ties to the lower index)."""
    inp = _grid(T, D, E, k, seed=5)
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, None, k)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    srt = -np.sort(-logits.astype(np.float64), axis=1)
    if k < E:
        assert np.array_equal(margin, srt[:, k - 1] - srt[:, k])
    else:
        assert np.all(np.isinf(margin))


def test_exact_ties_go_to_lower_index():
    """Grid inputs with few distinct values produce exact ties; the lower expert index wins."""
    s = W.Shape(T=200, D=8, E=16, k=4, F=8)
    inp = W.make_grid_inputs(s, seed=7)
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, None, s.k)
    assert np.any(margin == 0.0), "fixture must contain exact ties"
    for t in range(s.T):
        sel = ids[t]
        worst = logits[t, sel[-1]]
        # every unchosen expert tied with the k-th chosen has a larger index than it
        tied = [e for e in range(s.E) if e not in sel and logits[t, e] == worst]
        assert all(e > sel[-1] for e in tied)
        # slots are in descending logit order, ties by ascending index
        for j in range(s.k - 1):
            a, b = sel[j], sel[j + 1]
            assert logits[t, a] > logits[t, b] or (logits[t, a] == logits[t, b] and a < b)


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_weights_sum_to_one_and_match_softmax_then_renormalise(k):
    s = W.Shape(T=64, D=256, E=32, k=k, F=8)
    inp = W.make_inputs(s, seed=13)
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, None, k)
    assert np.all(np.abs(p.sum(1) - 1.0) <= 4 * k * 2.0 ** -52)
    # softmax over all E, restricted to the chosen, renormalised: the same weights
    full = sps.softmax(logits.astype(np.float64), axis=1)
    sub = np.take_along_axis(full, ids, axis=1)
    sub = sub / sub.sum(1, keepdims=True)
    assert np.max(np.abs(sub - p)) < 1e-12
    # slot 0 carries the largest weight
    assert np.all(p[:, 0] >= p.max(1) - 1e-15)


def test_k1_weight_is_exactly_one():
    s = W.Shape(T=64, D=128, E=8, k=1, F=8)
    inp = W.make_inputs(s, seed=2)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, None, 1)
    assert np.all(p == 1.0)


def test_shift_invariance():
    """A constant added to every logit changes neither the choice nor the weights."""
    s = W.Shape(T=64, D=64, E=16, k=4, F=8)
    inp = W.make_grid_inputs(s, seed=9)
    ids0, p0, _, l0 = oracle.route(inp.x, inp.w_g, None, s.k)
    bias = torch.full((s.E,), 0.375, dtype=torch.float32)  # exact on the grid
    ids1, p1, _, l1 = oracle.route(inp.x, inp.w_g, bias, s.k)
    assert np.array_equal(l1, l0 + np.float32(0.375))
    assert np.array_equal(ids0, ids1)
    assert np.max(np.abs(p0 - p1)) < 1e-15


def test_k_equals_E_selects_every_expert():
    s = W.Shape(T=16, D=64, E=6, k=6, F=8)
    inp = W.make_inputs(s, seed=4)
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, None, s.k)
    assert np.all(np.sort(ids, 1) == np.arange(6)[None, :])
    assert np.max(np.abs(p - np.take_along_axis(sps.softmax(logits.astype(np.float64), 1), ids, 1))) < 1e-12


def test_bias_steers_selection():
    """The skewed workload's bias b_e = -3.6 ln(e+1) shifts loads towards low experts."""
    s = W.Shape(T=2048, D=512, E=8, k=2, F=8, router_bias=True)
    inp = W.make_inputs(s, seed=0)
    ids, _, _, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, s.k)
    _, _, _, l_nobias = oracle.route(inp.x, inp.w_g, None, s.k)
    expect = (l_nobias.astype(np.float64) + inp.router_bias.double().numpy()[None]).astype(np.float32)
    assert np.max(np.abs(logits - expect)) <= 2.0 ** -22 * np.max(np.abs(expect))
    load = np.bincount(ids.ravel(), minlength=8) / ids.size
    assert load[0] > 0.4 and load[0] > load[1] > load[2]
