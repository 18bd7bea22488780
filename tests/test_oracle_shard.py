"""Pins of the oracle's expert-parallel shard (one call holds a contiguous
slice of the experts; only slots routed to them contribute).

"Mixture of Experts optimiza Transformers y LLMs", section "Expert
Parallelism", and "Transformers v5 El Secreto Detrás de los Modelos MoE Más
Rápidos", section "Paralelismo de Expertos": experts are distributed over
devices, every token's chosen experts run where they live, and the partial
results are added.  The dense reference below restricts its gate matrix to
the shard's experts: an implementation independent of the oracle's loop.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.dense_ref import dense_routing, f64, swiglu_ffn


def _slice(inp, e0, n, with_shared):
    """Inputs of one shard: experts e0 .. e0+n-1, the shared expert only if asked."""
    return W.LayerInputs(inp.shape if with_shared else dataclasses.replace(inp.shape, Fs=0),
                         inp.x, inp.w_g, inp.w_gate_up[e0:e0 + n].contiguous(),
                         inp.w_down[e0:e0 + n].contiguous(), inp.router_bias,
                         inp.ws_gate_up if with_shared else None,
                         inp.ws_down if with_shared else None)


def _dense_shard(inp, e0, n, with_shared):
    s = inp.shape
    ids, p, _ = dense_routing(inp)
    X = f64(inp.x)
    G = np.zeros((X.shape[0], s.E))
    np.put_along_axis(G, ids, p, axis=1)
    Y = np.zeros((X.shape[0], s.D))
    Wgu, Wd = f64(inp.w_gate_up), f64(inp.w_down)
    for e in range(e0, e0 + n):
        Y += G[:, e:e + 1] * swiglu_ffn(X, Wgu[e], Wd[e])
    if with_shared and s.Fs:
        Y += swiglu_ffn(X, f64(inp.ws_gate_up), f64(inp.ws_down))
    return Y


@pytest.mark.parametrize("T,D,E,k,F,Fs,bounds", [
    (40, 32, 8, 2, 16, 0, [0, 2, 5, 8]),
    (33, 64, 16, 4, 32, 16, [0, 4, 8, 12, 16]),
    (25, 32, 5, 5, 8, 0, [0, 1, 2, 3, 4, 5]),
])
def test_shards_add_up_to_the_layer(T, D, E, k, F, Fs, bounds):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T + E)
    y_full, ids, p, _ = oracle.forward(inp)
    total = np.zeros_like(y_full)
    for r, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        part = oracle.experts(_slice(inp, a, b - a, r == 0), ids, p, expert_begin=a, n_local=b - a)
        total += part
    scale = np.abs(y_full).max()
    assert np.max(np.abs(total - y_full)) <= 1e-12 * scale


@pytest.mark.parametrize("e0,n,with_shared", [(0, 2, True), (3, 3, False), (7, 1, False), (0, 8, True)])
def test_shard_matches_dense_restricted_gate(e0, n, with_shared):
    s = W.Shape(T=30, D=32, E=8, k=3, F=24, Fs=16)
    inp = W.make_inputs(s, seed=11)
    _, ids, p, _ = oracle.forward(inp)
    y = oracle.experts(_slice(inp, e0, n, with_shared), ids, p, expert_begin=e0, n_local=n)
    ref = _dense_shard(inp, e0, n, with_shared)
    scale = np.abs(ref).max()
    assert np.max(np.abs(y - ref)) <= 1e-10 * scale


def test_whole_range_shard_is_the_layer_bitwise():
    s = W.Shape(T=20, D=32, E=4, k=2, F=16, Fs=8)
    inp = W.make_inputs(s, seed=5)
    y_full, ids, p, _ = oracle.forward(inp)
    y = oracle.experts(inp, ids, p, expert_begin=0, n_local=4)
    assert np.array_equal(y, y_full)


def test_shard_without_routed_tokens_gives_zero_or_the_shared_expert():
    s = W.Shape(T=12, D=16, E=6, k=1, F=8, Fs=8, router_bias=True)
    inp = W.make_inputs(s, seed=2)
    inp.router_bias = torch.tensor([50.0, -50, -50, -50, -50, -50])  # every token picks expert 0
    _, ids, p, _ = oracle.forward(inp)
    assert np.all(ids == 0)
    y = oracle.experts(_slice(inp, 2, 3, False), ids, p, expert_begin=2, n_local=3)
    assert np.array_equal(y, np.zeros_like(y))
    y_sh = oracle.experts(_slice(inp, 2, 3, True), ids, p, expert_begin=2, n_local=3)
    ref = swiglu_ffn(f64(inp.x), f64(inp.ws_gate_up), f64(inp.ws_down))
    assert np.max(np.abs(y_sh - ref)) <= 1e-10 * np.abs(ref).max()


def test_shard_bounds_are_checked():
    s = W.Shape(T=4, D=16, E=4, k=2, F=8)
    inp = W.make_inputs(s, seed=1)
    _, ids, p, _ = oracle.forward(inp)
    with pytest.raises(ValueError):
        oracle.experts(_slice(inp, 3, 1, True), ids, p, expert_begin=3, n_local=2)
