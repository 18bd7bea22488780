"""moe_forward_noalloc (the entry point with its workspace in the library's
static per-GPU array) against moe_forward with a caller workspace, through
the C ABI: two calls in a row, the second with fewer tokens, each bitwise
equal to moe_forward on the same inputs (the same kernels run in both)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")

DEV = torch.device("cuda:0")


def _both(g, s, T, shard=None):
    """(noalloc outputs, moe_forward outputs) for the first T tokens; shard =
    (a, b) holds experts a .. b - 1 only (with their E4M3 scales if any)."""
    x = g.x[:T].contiguous()
    wgu, wd, eb = g.w_gate_up, g.w_down, None
    scales = None
    if s.fp8:
        scales = (g.w_gate_up_scale, g.w_down_scale, g.ws_gate_up_scale, g.ws_down_scale)
    if shard:
        a, b = shard
        wgu, wd, eb = wgu[a:b].contiguous(), wd[a:b].contiguous(), a
        if scales:
            scales = (scales[0][a:b].contiguous(), scales[1][a:b].contiguous(), scales[2], scales[3])
    outs = []
    for noalloc in (True, False):
        y = torch.full((T, s.D), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.full((T, s.k), -7, dtype=torch.int32, device=DEV)
        w = torch.full((T, s.k), float("nan"), dtype=torch.float32, device=DEV)
        f = moe.moe_forward_noalloc if noalloc else moe.moe_forward
        f(x, g.w_g, wgu, wd, s.k, g.router_bias, g.ws_gate_up, g.ws_down, y=y, topk_ids=ids,
          topk_w=w, expert_begin=eb, scales=scales)
        torch.cuda.synchronize()
        outs.append((y.cpu(), ids.cpu(), w.cpu()))
    return outs


@pytest.mark.parametrize("name,T0,T1", [("gptoss_decode", 64, 9), ("tiny", 64, 17)])
def test_noalloc_equals_forward(name, T0, T1):
    s = W.WORKLOADS[name].shape.with_T(T0)
    g = W.make_inputs(s, seed=3).to(DEV)
    for T in (T0, T1):  # the second call sees the first call's leftovers in the array
        (y_a, ids_a, w_a), (y_b, ids_b, w_b) = _both(g, s, T)
        assert torch.equal(ids_a, ids_b), "%s T=%d: ids differ" % (name, T)
        assert torch.equal(w_a, w_b), "%s T=%d: weights differ" % (name, T)
        assert torch.isfinite(y_a).all()
        assert torch.equal(y_a, y_b), "%s T=%d: y differs (max %g)" % (
            name, T, (y_a - y_b).abs().max().item())


def test_noalloc_e4m3_shard_with_shared_expert():
    """E4M3 weights, experts 4 .. 11 of 16 and a shared expert: the no-allocation
    entry point runs the same kernels as moe_forward, again on two calls."""
    s = W.Shape(T=48, D=256, E=16, k=4, F=128, Fs=64, fp8=True)
    g = W.make_inputs(s, seed=5).to(DEV)
    for T in (48, 13):
        (y_a, ids_a, w_a), (y_b, ids_b, w_b) = _both(g, s, T, shard=(4, 12))
        assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b), "T=%d: routing differs" % T
        assert torch.isfinite(y_a).all()
        assert torch.equal(y_a, y_b), "T=%d: y differs" % T
