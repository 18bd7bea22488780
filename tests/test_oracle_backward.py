"""Pins of the oracle's backward pass (gradients of sum_t <dy[t], y[t]>).

The pages' training sections name the backward only through its kernels
(grouped GEMMs), so the oracle is the chain rule of the forward function.  It
is pinned here against two independent derivations: torch's float64 autograd
of a dense formulation (a library derivative), and central finite differences
of a separate float64 numpy forward, plus closed-form special cases.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

TAG_DY = 99  # stream of the upstream gradient draws


def _inputs(T, D, E, k, F, Fs=0, seed=0, bias=False, select=False):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=bias, bias_select=select)
    return W.make_inputs(s, seed=seed)


def _dy(T, D, seed):
    return W.normal_f32((T, D), seed, TAG_DY, 1.0).numpy()


def _route(inp):
    s = inp.shape
    ids, p, margin, _ = oracle.route(inp.x, inp.w_g, inp.router_bias, s.k, select_only=s.bias_select)
    return ids, p, margin


def _autograd(inp, ids, dy):
    """torch float64 autograd of sum <dy, y>, the routing ids held fixed.  The
    logits are rounded to fp32 with an identity derivative, as the oracle's
    weights are a softmax of fp32 logits."""
    s = inp.shape
    X = inp.x.double().requires_grad_()
    Wg = inp.w_g.double().requires_grad_()
    in_logits = inp.router_bias is not None and not s.bias_select
    b = inp.router_bias.double().requires_grad_() if in_logits else None
    Wgu = inp.w_gate_up.double().requires_grad_()
    Wdn = inp.w_down.double().requires_grad_()
    l = X @ Wg.T + (b if b is not None else 0)
    l = l + (l.float().double() - l).detach()
    idx = torch.from_numpy(ids).long()
    p = torch.softmax(torch.gather(l, 1, idx), dim=1)
    y = torch.zeros(X.shape[0], s.D, dtype=torch.float64)
    for e in range(s.E):
        g = X @ Wgu[e, :s.F].T
        u = X @ Wgu[e, s.F:].T
        o = (torch.nn.functional.silu(g) * u) @ Wdn[e].T
        y = y + (p * (idx == e)).sum(1, keepdim=True) * o
    shared = []
    if s.Fs:
        Sgu = inp.ws_gate_up.double().requires_grad_()
        Sdn = inp.ws_down.double().requires_grad_()
        y = y + (torch.nn.functional.silu(X @ Sgu[:s.Fs].T) * (X @ Sgu[s.Fs:].T)) @ Sdn.T
        shared = [Sgu, Sdn]
    (y * torch.from_numpy(dy).double()).sum().backward()
    out = dict(dx=X.grad, dw_g=Wg.grad, dw_gate_up=Wgu.grad, dw_down=Wdn.grad,
               d_bias=b.grad if b is not None else torch.zeros(s.E, dtype=torch.float64))
    if s.Fs:
        out["dws_gate_up"], out["dws_down"] = shared[0].grad, shared[1].grad
    return {k_: v.numpy() for k_, v in out.items()}


CASES = [
    (12, 32, 8, 2, 24, 0, False, False),
    (9, 16, 5, 3, 8, 16, False, False),   # shared expert
    (10, 24, 6, 2, 16, 0, True, False),   # bias inside the logits: it gets a gradient
    (10, 24, 6, 2, 16, 0, True, True),    # selection-only bias: none
    (7, 16, 4, 4, 8, 0, False, False),    # k = E
]


@pytest.mark.parametrize("T,D,E,k,F,Fs,bias,select", CASES)
def test_matches_float64_autograd(T, D, E, k, F, Fs, bias, select):
    inp = _inputs(T, D, E, k, F, Fs, seed=T + D, bias=bias, select=select)
    ids, p, _ = _route(inp)
    dy = _dy(T, D, seed=T)
    mine = oracle.backward(inp, ids, p, dy)
    ref = _autograd(inp, ids, dy)
    for name, v in ref.items():
        scale = max(np.abs(v).max(), 1e-30)
        assert np.max(np.abs(mine[name] - v)) <= 1e-9 * scale, name
    if bias and select:
        assert np.all(mine["d_bias"] == 0)


def _np_loss(x, wg, b, wgu, wdn, sgu, sdn, ids, dy, F, Fs):
    """A separate float64 forward (fixed routing, no fp32 rounding)."""
    l = x @ wg.T + (b if b is not None else 0)
    lc = np.take_along_axis(l, ids, 1)
    pc = np.exp(lc - lc.max(1, keepdims=True))
    pc /= pc.sum(1, keepdims=True)
    y = np.zeros((x.shape[0], wdn.shape[1]))
    for t in range(x.shape[0]):
        for j in range(ids.shape[1]):
            e = ids[t, j]
            g, u = wgu[e, :F] @ x[t], wgu[e, F:] @ x[t]
            y[t] += pc[t, j] * (wdn[e] @ (g / (1 + np.exp(-g)) * u))
        if Fs:
            g, u = sgu[:Fs] @ x[t], sgu[Fs:] @ x[t]
            y[t] += sdn @ (g / (1 + np.exp(-g)) * u)
    return float((y * dy).sum())


def test_central_differences():
    T, D, E, k, F, Fs = 6, 12, 4, 2, 8, 8
    inp = _inputs(T, D, E, k, F, Fs, seed=3, bias=True)
    ids, p, margin = _route(inp)
    dy = _dy(T, D, seed=4).astype(np.float64)
    g = oracle.backward(inp, ids, p, dy.astype(np.float32))
    P = dict(x=inp.x.double().numpy(), wg=inp.w_g.double().numpy(),
             b=inp.router_bias.double().numpy(), wgu=inp.w_gate_up.double().numpy(),
             wdn=inp.w_down.double().numpy(), sgu=inp.ws_gate_up.double().numpy(),
             sdn=inp.ws_down.double().numpy())
    grads = dict(x="dx", wg="dw_g", b="d_bias", wgu="dw_gate_up", wdn="dw_down", sgu="dws_gate_up",
                 sdn="dws_down")
    rng = np.random.default_rng(0)
    eps = 1e-5
    for name, gname in grads.items():
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in P[name].shape)
            vals = []
            for sgn in (1, -1):
                Q = {k_: v.copy() for k_, v in P.items()}
                Q[name][idx] += sgn * eps
                vals.append(_np_loss(Q["x"], Q["wg"], Q["b"], Q["wgu"], Q["wdn"], Q["sgu"], Q["sdn"],
                                     ids, dy, F, Fs))
            fd = (vals[0] - vals[1]) / (2 * eps)
            an = g[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_single_expert_has_no_router_gradient():
    """E = k = 1: p is identically 1, so the router gets exactly zero."""
    inp = _inputs(8, 16, 1, 1, 8, seed=2, bias=True)
    ids, p, _ = _route(inp)
    g = oracle.backward(inp, ids, p, _dy(8, 16, 5))
    assert np.all(g["dw_g"] == 0) and np.all(g["d_bias"] == 0)


def test_unchosen_expert_gets_exactly_zero():
    inp = _inputs(16, 32, 8, 2, 16, seed=6)
    ids, p, _ = _route(inp)
    ids[ids == 5] = 6  # no token uses expert 5 (a valid routing of its own)
    ids = np.where(ids[:, :1] == ids[:, 1:], np.stack([ids[:, 0], (ids[:, 0] + 1) % 5], 1), ids)
    assert not np.any(ids == 5)
    g = oracle.backward(inp, ids, p, _dy(16, 32, 7))
    assert np.all(g["dw_gate_up"][5] == 0) and np.all(g["dw_down"][5] == 0)
    assert np.all(g["dw_g"][5] == 0)


def test_linear_in_dy():
    inp = _inputs(10, 16, 4, 2, 8, 8, seed=8)
    ids, p, _ = _route(inp)
    dy = _dy(10, 16, 9)
    g1 = oracle.backward(inp, ids, p, dy)
    g2 = oracle.backward(inp, ids, p, 2 * dy)
    for name in g1:
        assert np.array_equal(g2[name], 2 * g1[name]), name


def test_dp_is_the_slot_output_projection():
    """dp[t,j] = <dy[t], O_j>: weighting the experts' outputs by dp reproduces
    sum_j p_j dp_j = <dy, y - shared>."""
    inp = _inputs(8, 16, 4, 2, 8, seed=10)
    ids, p, _ = _route(inp)
    dy = _dy(8, 16, 11)
    g = oracle.backward(inp, ids, p, dy)
    y = oracle.experts(inp, ids, p)
    assert np.allclose((p * g["dp"]).sum(1), (y * dy.astype(np.float64)).sum(1), rtol=1e-12, atol=1e-14)
