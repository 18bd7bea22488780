"""GPU parity of the backward pass (moe_backward) against the oracle's gradients.

Every call goes through the C ABI.  Each gradient tensor g is compared with
the oracle's float64 gradient g0 on two norms, relative to RMS(g0):
RMS(g - g0) <= GRAD_RMS_TOL (1%) and max|g - g0| <= GRAD_MAX_TOL (15%).  The
gradient GEMMs take bf16 operands (dy, h, dg, du; x is bf16 already) with fp32
accumulation; tests/test_tolerances.py emulates exactly these roundings on
every case here and derives both bars from them (RMS errors of 0.2-0.3%, and
up to 11% on the largest entries of dW_down, whose rows sum as few as one
heavy-tailed routed token).  A lost or doubled row, a wrong weight or a wrong
sign moves the RMS error by several percent and fails the first norm.

d_bias is a sum over tokens of terms of either sign, and its value can cancel
far below the size of those terms (one seed here gives 0.05 where the terms'
root-sum-square is 1.5, other dy draws give 0.3 to 2.5).  Its errors are those
of the terms, so its scale is the root-sum-square of its terms when that is
larger than its own RMS.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import tolerances as TL

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")
DEV = torch.device("cuda:0")
TAG_DY = 99
RMS_TOL, MAX_TOL = TL.GRAD_RMS_TOL, TL.GRAD_MAX_TOL
grad_error = TL.grad_error


def bias_terms_scale(ref, ids, p, E):
    return TL.bias_terms_scale(ref["dp"], ids, p, E)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.load_library()


def _run(inp, seed=0, workspace=None):
    s = inp.shape
    T = inp.x.shape[0]
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, inp.router_bias, s.k, select_only=s.bias_select)
    p32 = p.astype(np.float32)
    dy = W.normal_f32((T, s.D), seed, TAG_DY, 1.0)
    g = inp.to(DEV)
    out = moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, torch.from_numpy(ids).to(DEV),
                           torch.from_numpy(p32).to(DEV), dy.to(DEV), g.router_bias, g.ws_gate_up,
                           g.ws_down, bias_select=s.bias_select, workspace=workspace)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}, ids, p32, dy.numpy()


CASES = [
    (64, 128, 8, 2, 256, 0, False),      # 16-row tiles
    (300, 512, 64, 8, 256, 256, False),  # 32-row tiles, shared expert
    (40, 200, 8, 2, 136, 0, True),       # 16-row tiles, ragged K, bias in the logits
    (2048, 256, 8, 2, 512, 0, False),    # 256-row tiles
    (1500, 320, 8, 2, 200, 0, True),     # 256-row tiles, ragged M, N and K, bias in the logits
    (700, 512, 16, 4, 256, 256, False),  # 256-row tiles with the shared expert
    (32, 1024, 8, 2, 768, 256, False),   # 16-row tiles, K = 1024 and 1536: several K chunks per wave
    (200, 1024, 16, 2, 640, 0, True),    # 32-row tiles, K = 1024 and 1280
    (200, 200, 16, 2, 136, 64, False),   # 32-row tiles, ragged K and N, shared expert
    # T <= 64: the weight gradients' one-stage kernel, several tiles per workgroup
    (64, 2048, 16, 2, 1024, 0, False),
    # weight-staging 16/32-row tiles on ragged shapes (N % 32 = 8, K % 64 = 40):
    # the g | u recomputation (N = 2F = 2000) and the K-major products
    (64, 1000, 32, 4, 1000, 0, False),
    (256, 1000, 64, 8, 1000, 136, False),
]


def test_backward_cases_reach_the_staged_tiles():
    from tests.test_gpu_kernels import staged_decode_tiles
    assert staged_decode_tiles(64, 1000, 32, 4, 1000, 0)
    assert staged_decode_tiles(256, 1000, 64, 8, 1000, 136)


@pytest.mark.parametrize("T,D,E,k,F,Fs,bias", CASES)
def test_backward_parity(T, D, E, k, F, Fs, bias):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=bias)
    inp = W.make_inputs(s, seed=T + F)
    got, ids, p32, dy = _run(inp, seed=T)
    ref = oracle.backward(inp, ids, p32.astype(np.float64), dy)
    for name in got:
        if name == "d_bias" and not bias:
            assert np.all(got[name] == 0)
            continue
        sc = bias_terms_scale(ref, ids, p32.astype(np.float64), E) if name == "d_bias" else 0.0
        r, m = grad_error(got[name], ref[name], sc)
        print("T=%d D=%d E=%d k=%d F=%d Fs=%d %s: RMS err %.3g, max err %.3g (of RMS)" % (
            T, D, E, k, F, Fs, name, r, m))
        assert r <= RMS_TOL and m <= MAX_TOL, name


def test_backward_selection_bias_gets_no_gradient():
    s = W.Shape(T=64, D=256, E=8, k=2, F=128, router_bias=True, bias_select=True)
    inp = W.make_inputs(s, seed=3)
    got, ids, p32, dy = _run(inp, seed=1)
    assert np.all(got["d_bias"] == 0)
    ref = oracle.backward(inp, ids, p32.astype(np.float64), dy)
    r, m = grad_error(got["dw_g"], ref["dw_g"])
    assert r <= RMS_TOL and m <= MAX_TOL


def test_backward_deterministic_with_poisoned_workspace():
    """Two calls, the second on a workspace full of 0xFF bytes: bitwise equal."""
    s = W.Shape(T=1024, D=256, E=8, k=2, F=512, Fs=128)
    inp = W.make_inputs(s, seed=5)
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, s.Fs)
    ws = torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device=DEV)
    a, _, _, _ = _run(inp, seed=2, workspace=ws)
    ws.fill_(0xFF)
    b, _, _, _ = _run(inp, seed=2, workspace=ws)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


def test_backward_zero_tokens():
    s = W.Shape(T=0, D=128, E=4, k=2, F=64, Fs=64)
    inp = W.make_inputs(s, seed=1)
    g = inp.to(DEV)
    grads = {n: torch.full(shp, 7.0, device=DEV) for n, shp in
             dict(dx=(0, 128), dw_g=(4, 128), d_bias=(4,), dw_gate_up=(4, 128, 128),
                  dw_down=(4, 128, 64), dws_gate_up=(128, 128), dws_down=(128, 64)).items()}
    out = moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, 2,
                           torch.empty((0, 2), dtype=torch.int32, device=DEV),
                           torch.empty((0, 2), device=DEV), torch.empty((0, 128), device=DEV),
                           None, g.ws_gate_up, g.ws_down, grads=grads)
    torch.cuda.synchronize()
    for name, v in out.items():
        assert torch.all(v == 0), name


TRAIN_CASES = [
    (64, 128, 8, 2, 256, 0, False),      # 16-row tiles
    (300, 512, 64, 8, 256, 256, False),  # 32-row tiles, shared expert
    (1500, 320, 8, 2, 200, 0, True),     # 256-row tiles, ragged M, N and K, bias in the logits
    (700, 512, 16, 4, 256, 256, False),  # 256-row tiles with the shared expert
    (4096, 512, 8, 2, 384, 0, False),    # 256-row tiles, more tiles than run at once
    (270, 256, 2, 2, 320, 64, False),    # every group 270 rows: 14 folded into the first tile
]


@pytest.mark.parametrize("T,D,E,k,F,Fs,bias", TRAIN_CASES)
def test_forward_train_then_backward_saved(T, D, E, k, F, Fs, bias):
    """moe_forward_train returns moe_forward's results bitwise; the backward on
    its saved g | u (bf16) meets the same bar against the oracle, and stays
    within the bar of the backward that recomputes g | u in fp32."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=bias)
    inp = W.make_inputs(s, seed=T + F + 1)
    g = inp.to(DEV)
    ids0 = torch.empty((T, k), dtype=torch.int32, device=DEV)
    p0 = torch.empty((T, k), dtype=torch.float32, device=DEV)
    y0 = moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, k, g.router_bias, g.ws_gate_up, g.ws_down,
                         topk_ids=ids0, topk_w=p0)
    y, ids, p, saved = moe.moe_forward_train(g.x, g.w_g, g.w_gate_up, g.w_down, k, g.router_bias,
                                             g.ws_gate_up, g.ws_down)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(ids, ids0) and torch.equal(p, p0)
    dy = W.normal_f32((T, D), T, TAG_DY, 1.0)
    dyd = dy.to(DEV)
    args = (g.x, g.w_g, g.w_gate_up, g.w_down, k, ids, p, dyd, g.router_bias, g.ws_gate_up, g.ws_down)
    got = {n: v.cpu().numpy() for n, v in moe.moe_backward(*args, saved=saved).items()}
    again = {n: v.cpu().numpy() for n, v in moe.moe_backward(*args).items()}
    ids_h, p_h = ids.cpu().numpy(), p.cpu().numpy().astype(np.float64)
    ref = oracle.backward(inp, ids_h, p_h, dy.numpy())
    for name in got:
        if name == "d_bias" and not bias:
            assert np.all(got[name] == 0)
            continue
        sc = bias_terms_scale(ref, ids_h, p_h, E) if name == "d_bias" else 0.0
        r, m = grad_error(got[name], ref[name], sc)
        r2, m2 = grad_error(got[name], again[name].astype(np.float64), sc)
        print("T=%d %s: vs oracle RMS %.3g max %.3g; vs recompute RMS %.3g max %.3g" % (
            T, name, r, m, r2, m2))
        assert r <= RMS_TOL and m <= MAX_TOL, name
        assert r2 <= RMS_TOL and m2 <= MAX_TOL, name


def test_backward_saved_twice_is_deterministic():
    """The saved workspace is read only: two backward calls on it, the second
    on a poisoned backward workspace, are bitwise equal."""
    s = W.Shape(T=1024, D=256, E=8, k=2, F=512, Fs=128)
    inp = W.make_inputs(s, seed=9)
    g = inp.to(DEV)
    _, ids, p, saved = moe.moe_forward_train(g.x, g.w_g, g.w_gate_up, g.w_down, 2, None,
                                             g.ws_gate_up, g.ws_down)
    dy = W.normal_f32((1024, 256), 3, TAG_DY, 1.0).to(DEV)
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, s.Fs)
    ws = torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device=DEV)
    args = (g.x, g.w_g, g.w_gate_up, g.w_down, 2, ids, p, dy, None, g.ws_gate_up, g.ws_down)
    a = {n: v.clone() for n, v in moe.moe_backward(*args, saved=saved, workspace=ws).items()}
    ws.fill_(0xFF)
    b = moe.moe_backward(*args, saved=saved, workspace=ws)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("counts,D,F", [
    ([257, 300, 511, 512, 256, 1, 0, 700], 256, 320),  # 256-row tiles
    # 256-row tiles whose groups' last few rows fold into the tile before (270,
    # 288, 513, 1030 rows; the shared expert's 2456 = 9 * 256 + 152 do not)
    ([270, 288, 289, 513, 1030, 0, 40, 26], 136, 200),
    ([16, 17, 1, 0, 15, 32, 8, 3], 256, 320),          # 16-row tiles
    ([33, 32, 64, 1, 0, 40, 31, 47], 256, 320),        # 32-row tiles
    # T = 64: the one-stage weight gradients, 576 tiles over 256 workgroups, with
    # empty groups' tiles between others in a workgroup's sequence
    ([9, 0, 13, 1, 0, 7, 20, 14], 2048, 1024),
])
def test_backward_tile_boundaries(counts, D, F):
    """The backward's tiles at group sizes around tile boundaries (k = 1, exact
    counts, tokens shuffled), with a shared expert.  With k = 1 the routing weight
    is 1 and the router gradient is exactly 0."""
    T, E = sum(counts), len(counts)
    s = W.Shape(T=T, D=D, E=E, k=1, F=F, Fs=64)
    inp = W.make_inputs(s, seed=12)
    order = np.random.default_rng(6).permutation(T)
    ids = np.repeat(np.arange(E), counts)[order].astype(np.int32).reshape(T, 1)
    p32 = np.ones((T, 1), np.float32)
    dy = W.normal_f32((T, D), 3, TAG_DY, 1.0)
    g = inp.to(DEV)
    got = moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, 1, torch.from_numpy(ids).to(DEV),
                           torch.from_numpy(p32).to(DEV), dy.to(DEV), None, g.ws_gate_up, g.ws_down)
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in got.items()}
    ref = oracle.backward(inp, ids, p32.astype(np.float64), dy.numpy())
    assert np.all(got["dw_g"] == 0) and np.all(got["d_bias"] == 0)
    z = counts.index(0)  # the empty expert
    assert np.all(got["dw_gate_up"][z] == 0) and np.all(got["dw_down"][z] == 0)
    for name in ("dx", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"):
        r, m = grad_error(got[name], ref[name])
        print("tile boundaries %s: RMS err %.3g, max err %.3g (of RMS)" % (name, r, m))
        assert r <= RMS_TOL and m <= MAX_TOL, name
