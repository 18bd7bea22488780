"""The layer inside a captured HIP graph: every replay must equal an eager call.

Each test captures a call once, then replays it three times with new inputs
written eagerly between the replays (and a synchronisation), and compares each
replay bit for bit with an eager call on the same inputs and its own buffers.
The library enqueues only kernels (no memsets), so replays stay exact.
"""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.load_library()


@pytest.mark.parametrize("T,D,E,k,F,Fs", [(64, 2880, 32, 4, 512, 0), (1024, 512, 8, 2, 512, 256)])
def test_forward_graph_replays_match_eager(T, D, E, k, F, Fs):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    g = W.make_inputs(s, seed=T).to(DEV)
    x = g.x.clone()
    shape = moe.make_shape(T, D, E, F, k, Fs)
    ws = moe.alloc_workspace(shape, DEV)
    y = torch.empty((T, D), device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), device=DEV)

    def fwd(xx, yy, ii, ww, wsp):
        moe.moe_forward(xx, g.w_g, g.w_gate_up, g.w_down, k, None, g.ws_gate_up, g.ws_down, y=yy,
                        topk_ids=ii, topk_w=ww, workspace=wsp)

    fwd(x, y, ids, w, ws)  # first call outside the graph (one-time kernel attributes)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(x, y, ids, w, ws)
    ws2 = moe.alloc_workspace(shape, DEV)
    for r in range(3):
        x.copy_(W.make_x(T, D, seed=100 + r).to(DEV))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y2 = torch.empty_like(y)
        ids2 = torch.empty_like(ids)
        w2 = torch.empty_like(w)
        fwd(x, y2, ids2, w2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids2) and torch.equal(w, w2), r
        assert torch.equal(y, y2), r


def test_backward_graph_replays_match_eager():
    T, D, E, k, F, Fs = 512, 256, 8, 2, 256, 128
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    g = W.make_inputs(s, seed=7).to(DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), device=DEV)
    moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, k, None, g.ws_gate_up, g.ws_down, topk_ids=ids,
                    topk_w=w)
    dy = W.normal_f32((T, D), 1, 99, 1.0).to(DEV)
    shape = moe.make_shape(T, D, E, F, k, Fs)
    ws = torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device=DEV)

    def bwd(wsp, grads=None):
        return moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, k, ids, w, dy, None, g.ws_gate_up,
                                g.ws_down, workspace=wsp, grads=grads)

    grads = bwd(ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bwd(ws, grads)
    ws2 = torch.empty_like(ws)
    for r in range(3):
        dy.copy_(W.normal_f32((T, D), 10 + r, 99, 1.0).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = bwd(ws2)
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(grads[name], ref[name]), (r, name)


def test_training_step_graph_replays_match_eager():
    """moe_forward_train then moe_backward_saved, captured together as one step."""
    T, D, E, k, F, Fs = 700, 256, 8, 2, 256, 128
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    g = W.make_inputs(s, seed=8).to(DEV)
    x = g.x.clone()
    dy = W.normal_f32((T, D), 2, 99, 1.0).to(DEV)
    shape = moe.make_shape(T, D, E, F, k, Fs)

    def bufs():
        return dict(y=torch.empty((T, D), device=DEV),
                    ids=torch.empty((T, k), dtype=torch.int32, device=DEV),
                    w=torch.empty((T, k), device=DEV),
                    tws=torch.empty(moe.train_workspace_size(shape), dtype=torch.uint8, device=DEV),
                    bws=torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device=DEV),
                    grads=None)

    def step(b):
        moe.moe_forward_train(x, g.w_g, g.w_gate_up, g.w_down, k, None, g.ws_gate_up, g.ws_down,
                              y=b["y"], topk_ids=b["ids"], topk_w=b["w"], workspace=b["tws"])
        b["grads"] = moe.moe_backward(x, g.w_g, g.w_gate_up, g.w_down, k, b["ids"], b["w"], dy, None,
                                      g.ws_gate_up, g.ws_down, workspace=b["bws"],
                                      grads=b["grads"], saved=b["tws"])

    a = bufs()
    step(a)  # allocates the gradients and sets the kernels' attributes outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(a)
    ref = bufs()
    for r in range(3):
        x.copy_(W.make_x(T, D, seed=200 + r).to(DEV))
        dy.copy_(W.normal_f32((T, D), 20 + r, 99, 1.0).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(ref)
        torch.cuda.synchronize()
        assert torch.equal(a["y"], ref["y"]) and torch.equal(a["ids"], ref["ids"]), r
        for name in ref["grads"]:
            assert torch.equal(a["grads"][name], ref["grads"][name]), (r, name)
