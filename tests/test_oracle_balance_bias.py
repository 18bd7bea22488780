"""Pins of the oracle's selection-only router bias (auxiliary-loss-free balancing).

The glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 2 item 4,
names a load balancer that works without an auxiliary loss by adjusting
per-expert router biases.  Reading taken: the bias is added to the fp32 logit
for the top-k selection only (key = fp32(l + b)); the weights are the softmax
over the plain logits of the chosen experts, so the bias steers which experts
run and never how much each contributes.
"""
import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import workloads as W
from tests.dense_ref import dense_forward, dense_routing


def _inputs(T, D, E, k, seed=0, Fs=0, F=8):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=True, bias_select=True)
    return W.make_inputs(s, seed=seed)


def test_zero_bias_is_the_plain_router():
    s = W.Shape(T=96, D=256, E=32, k=4, F=8)
    inp = W.make_inputs(s, seed=1)
    ids0, p0, m0, l0 = oracle.route(inp.x, inp.w_g, None, s.k)
    zero = torch.zeros(s.E, dtype=torch.float32)
    ids1, p1, m1, l1 = oracle.route(inp.x, inp.w_g, zero, s.k, select_only=True)
    assert np.array_equal(ids0, ids1) and np.array_equal(p0, p1)
    assert np.array_equal(m0, m1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("T,D,E,k", [(128, 256, 8, 2), (64, 128, 32, 4), (24, 64, 256, 8), (16, 32, 6, 6)])
def test_selection_and_weights_match_dense(T, D, E, k):
    """Against the dense reference (stable argsort of the fp32 keys, scipy
    softmax of the chosen plain logits); ids compared where the key margin
    leaves no room for a rounding-order flip."""
    inp = _inputs(T, D, E, k, seed=E)
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, k, select_only=True)
    ids_d, p_d, l_d = dense_routing(inp)
    safe = margin > 1e-5
    assert safe.mean() > 0.9
    assert np.array_equal(ids[safe], ids_d[safe])
    assert np.max(np.abs(p[safe] - p_d[safe])) < 1e-6
    assert np.max(np.abs(logits.astype(np.float64) - l_d)) < 1e-5


def test_margin_is_the_key_gap():
    inp = _inputs(64, 128, 16, 3, seed=4)
    ids, _, margin, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, 3, select_only=True)
    key = (logits + inp.router_bias.numpy()[None, :]).astype(np.float64)
    srt = -np.sort(-key, axis=1)
    assert np.array_equal(margin, srt[:, 2] - srt[:, 3])
    # the chosen are the three largest keys, slot order by key
    assert np.array_equal(np.take_along_axis(key, ids, 1), srt[:, :3])


def test_weights_depend_only_on_the_chosen_set():
    """Scaling the bias changes the weights only through the chosen set: for
    every token whose set is unchanged the weights stay the same."""
    inp = _inputs(256, 128, 16, 4, seed=7)
    b = inp.router_bias
    ids1, p1, _, l1 = oracle.route(inp.x, inp.w_g, b, 4, select_only=True)
    ids2, p2, _, _ = oracle.route(inp.x, inp.w_g, b * 1.25, 4, select_only=True)
    o1, o2 = np.argsort(ids1, 1), np.argsort(ids2, 1)  # compare per expert id
    s1, s2 = np.take_along_axis(ids1, o1, 1), np.take_along_axis(ids2, o2, 1)
    same = np.all(s1 == s2, axis=1)
    changed = ~same
    assert same.sum() > 50 and changed.sum() > 10
    q1, q2 = np.take_along_axis(p1, o1, 1), np.take_along_axis(p2, o2, 1)
    # the same terms summed in another slot order: equal up to the sum's rounding
    assert np.max(np.abs(q1[same] - q2[same])) < 1e-15
    # and they are the softmax of the plain logits at the chosen ids
    ref = sps.softmax(np.take_along_axis(l1.astype(np.float64), ids1, 1), axis=1)
    assert np.max(np.abs(p1 - ref)) < 1e-15


def test_large_bias_forces_an_expert_but_not_its_weight():
    """A +1000 bias on expert 3 puts it in slot 0 of every token; its weight is
    still the softmax of plain logits, unlike a bias inside the logits (which
    gives it weight ~1)."""
    s = W.Shape(T=200, D=128, E=8, k=2, F=8)
    inp = W.make_inputs(s, seed=3)
    b = torch.zeros(8, dtype=torch.float32)
    b[3] = 1000.0
    ids, p, _, l = oracle.route(inp.x, inp.w_g, b, 2, select_only=True)
    assert np.all(ids[:, 0] == 3)
    l = l.astype(np.float64)
    other = ids[:, 1]
    assert np.all(np.take_along_axis(l, other[:, None], 1)[:, 0] == np.max(np.delete(l, 3, axis=1), axis=1))
    expect = 1.0 / (1.0 + np.exp(l[np.arange(200), other] - l[:, 3]))
    assert np.max(np.abs(p[:, 0] - expect)) < 1e-14
    assert p[:, 0].min() < 0.5  # the weight is not pinned at 1
    _, p_in, _, _ = oracle.route(inp.x, inp.w_g, b, 2, select_only=False)
    assert p_in[:, 0].min() > 1.0 - 1e-12


def test_k1_weight_is_exactly_one():
    inp = _inputs(64, 64, 8, 1, seed=2)
    _, p, _, _ = oracle.route(inp.x, inp.w_g, inp.router_bias, 1, select_only=True)
    assert np.all(p == 1.0)


def test_k_equals_E_weights_are_the_full_softmax():
    inp = _inputs(16, 64, 6, 6, seed=5)
    ids, p, margin, l = oracle.route(inp.x, inp.w_g, inp.router_bias, 6, select_only=True)
    assert np.all(np.sort(ids, 1) == np.arange(6)[None, :]) and np.all(np.isinf(margin))
    full = sps.softmax(l.astype(np.float64), axis=1)
    assert np.max(np.abs(p - np.take_along_axis(full, ids, 1))) < 1e-12


def test_balancing_bias_evens_out_the_load():
    """The use the glossary names: a bias against over-loaded experts evens the
    load.  One correction step b_e -= 2 * (load_e - mean) on a skewed router
    must lower the largest expert load."""
    s = W.Shape(T=2048, D=256, E=8, k=2, F=8)
    inp = W.make_inputs(s, seed=0)
    inp.x += 0.25       # a direction every token shares ...
    inp.w_g[0] += 0.02  # ... that expert 0 scores: it is in most tokens' top-2
    ids0, _, _, _ = oracle.route(inp.x, inp.w_g, None, 2)
    load0 = np.bincount(ids0.ravel(), minlength=8) / ids0.size
    assert load0.max() > 0.4
    b = torch.tensor(-2.0 * (load0 - load0.mean()), dtype=torch.float32)
    ids1, _, _, _ = oracle.route(inp.x, inp.w_g, b, 2, select_only=True)
    load1 = np.bincount(ids1.ravel(), minlength=8) / ids1.size
    assert load1.max() < load0.max() and load1.std() < load0.std()


def test_layer_matches_dense_forward():
    """The whole layer with a selection-only bias against the dense gate."""
    inp = _inputs(48, 64, 8, 2, seed=6, Fs=32, F=48)
    y, ids, p, margin = oracle.forward(inp)
    y_d, ids_d, p_d = dense_forward(inp)
    safe = margin > 1e-5
    assert safe.all()
    assert np.array_equal(ids, ids_d)
    assert np.max(np.abs(y - y_d)) < 1e-9 * max(1.0, np.abs(y_d).max())


def test_invalid_mode_rejected():
    lib = oracle._load()
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.zeros(4, 8, dtype=torch.bfloat16)
    out = np.zeros(64, np.float64)
    ids = np.zeros(16, np.int32)
    lg = np.zeros(16, np.float32)
    for bias, mode in [(None, 2), (None, 1), (torch.zeros(4), 0), (torch.zeros(4), 3)]:
        pb = None if bias is None else bias.data_ptr()
        rc = lib.oracle_route_mode(x.data_ptr(), w.data_ptr(), pb, mode, 4, 8, 4, 2, lg.ctypes.data,
                                   ids.ctypes.data, out.ctypes.data, out.ctypes.data)
        assert rc == -1
