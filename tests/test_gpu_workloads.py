"""GPU parity at the full sizes of the five named workloads, in the launch
configuration the benchmark times.

Routing and grouping are checked on every token.  The layer output is
checked on every token of the tiny, gpt-oss-shaped and Mixtral-shaped
workloads, and elsewhere on a deterministic sample the oracle computes one by
one: every (T/n)-th token, every near-tie token, and the tokens owning the
first and the last valid row of every m-tile of every expert group (so every
row tile of both GEMMs, the split pieces of a last round included, holds a
compared row).
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import (Y_TOL, align_equal, check_routing, reference_y, sample_tokens,
                          tile_edge_tokens, y_error)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")
DEV = torch.device("cuda:0")


def _run(name, T=None, n_sample=48, fp8=False):
    wl = W.WORKLOADS[name]
    s = wl.shape if T is None else wl.shape.with_T(T)
    if fp8:
        s = dataclasses.replace(s, fp8=True)
    t0 = time.time()
    inp = W.make_inputs(s, seed=0)
    g = inp.to(DEV)
    t_gen = time.time() - t0
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=DEV)
    w = torch.empty((s.T, s.k), dtype=torch.float32, device=DEV)
    scales = (g.w_gate_up_scale, g.w_down_scale, g.ws_gate_up_scale, g.ws_down_scale) if fp8 else None
    y = moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, g.router_bias, g.ws_gate_up,
                        g.ws_down, topk_ids=ids, topk_w=w, scales=scales)
    torch.cuda.synchronize()
    ids_g, w_g, y_g = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    del g, y
    t1 = time.time()
    ids_or, p_or, margin, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, s.k)
    flipped = check_routing(ids_g, w_g, ids_or, p_or, margin, logits, s.k)
    # grouping of the GPU's own routing, bit-exact against the oracle's grouping
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, s.Fs, s.router_bias,
                           weight_format=moe.WEIGHTS_FP8_E4M3 if fp8 else moe.WEIGHTS_BF16)
    bm = moe.moe_block_m(shape)
    out = moe.moe_align(torch.from_numpy(ids_g).to(DEV), s.E, bm, s.T if s.Fs else 0)
    ref = oracle.align(ids_g, s.E, bm, shared=bool(s.Fs))
    align_equal({k_: v.cpu().numpy() for k_, v in out.items()}, ref)
    # tokens owning the first and last valid row of every m-tile of every group
    edges = tile_edge_tokens(ref, bm)
    tok = sample_tokens(s.T, n_sample, list(flipped) + edges)
    y_ref = reference_y(inp, ids_or, p_or, ids_g, w_g, flipped, tok)
    rel, err, rms = y_error(y_g[tok], y_ref)
    loads = np.bincount(ids_g.ravel(), minlength=s.E)
    print("%s T=%d: gen %.1fs oracle %.1fs, compared %d tokens, max|err|/RMS=%.4g (err %.3g, rms %.3g), "
          "near-tie flips %d, max load %d, empty experts %d" % (
              name, s.T, t_gen, time.time() - t1, tok.size, rel, err, rms, len(flipped),
              loads.max(), int((loads == 0).sum())))
    assert rel <= Y_TOL
    return loads


def test_tiny_all_tokens():
    _run("tiny", n_sample=64)


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_gptoss_decode(T):
    _run("gptoss_decode", T=T, n_sample=64)


@pytest.mark.parametrize("T", [1, 64])
def test_gptoss_decode_fp8_weights(T):
    """The gpt-oss-shaped decode layer with E4M3 expert weights (per-row scales)."""
    _run("gptoss_decode", T=T, n_sample=64, fp8=True)


def test_mixtral_prefill():
    _run("mixtral_prefill", n_sample=4096)  # every token


def test_mixtral_prefill_fp8_weights():
    """The Mixtral-shaped prefill layer with E4M3 expert weights."""
    _run("mixtral_prefill", fp8=True)


def test_mixtral_skewed():
    loads = _run("mixtral_skewed")
    assert loads[0] > 0.4 * loads.sum()


def test_deepseek_fine():
    _run("deepseek_fine", n_sample=32)
