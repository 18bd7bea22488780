"""GPU parity of each kernel and of the layer, at sizes the oracle finishes in seconds.

Every call goes through the C ABI (libmoe.so) via the ctypes binding.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import tolerances as TL
from tests.parity import Y_TOL, align_equal, check_routing, reference_y, sample_tokens, y_error

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.load_library()  # raises loudly when libmoe.so is missing


def _gpu(inp):
    return inp.to(DEV)


def _forward(inp, **kw):
    g = _gpu(inp)
    s = inp.shape
    T = inp.x.shape[0]
    ids = torch.empty((T, s.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, s.k), dtype=torch.float32, device=DEV)
    y = moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, g.router_bias, g.ws_gate_up,
                        g.ws_down, topk_ids=ids, topk_w=w, bias_select=s.bias_select,
                        scales=_scales(g), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def _scales(g):
    """The row scales of E4M3 expert weights (None for bf16 weights)."""
    if not g.shape.fp8:
        return None
    return (g.w_gate_up_scale, g.w_down_scale, g.ws_gate_up_scale, g.ws_down_scale)


def _route_oracle(inp, k):
    """Oracle routing plus the values the selection is taken on (the logits,
    or logit + bias with a selection-only bias)."""
    sel = inp.shape.bias_select
    ids, p, margin, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, k, select_only=sel)
    keys = logits + inp.router_bias.numpy()[None, :] if sel else logits
    return ids, p, margin, keys


def _layer_parity(inp, tokens=None):
    s = inp.shape
    y, ids_g, w_g = _forward(inp)
    ids_or, p_or, margin, logits = _route_oracle(inp, s.k)
    flipped = check_routing(ids_g, w_g, ids_or, p_or, margin, logits, s.k)
    T = inp.x.shape[0]
    tok = np.arange(T) if tokens is None else tokens
    y_ref = reference_y(inp, ids_or, p_or, ids_g, w_g, flipped, tok)
    rel, err, rms = y_error(y[tok], y_ref)
    print("T=%d D=%d E=%d k=%d F=%d Fs=%d: max|err|/RMS=%.4g flips=%d" % (
        T, s.D, s.E, s.k, s.F, s.Fs, rel, len(flipped)))
    assert rel <= Y_TOL
    return y, ids_g, w_g


# --------------------------------------------------------------------- router
@pytest.mark.parametrize("T,D,E,k,bias", [
    (64, 128, 8, 2, False), (300, 2880, 32, 4, False), (97, 7168, 256, 8, False),
    (1, 64, 3, 3, False), (50, 4096, 8, 2, True), (33, 136, 17, 5, False),
    # E > 128 (two token tiles per workgroup, W_g column tiles loaded in pairs):
    # ragged expert count, and fewer K chunks than the workgroup has waves
    (300, 512, 129, 4, True), (40, 136, 200, 8, False)])
def test_router_parity(T, D, E, k, bias):
    s = W.Shape(T=T, D=D, E=E, k=k, F=8, router_bias=bias)
    inp = W.make_inputs(s, seed=T + D)
    g = _gpu(inp)
    ids, w = moe.moe_route(g.x, g.w_g, k, g.router_bias)
    torch.cuda.synchronize()
    ids_or, p_or, margin, logits = oracle.route(inp.x, inp.w_g, inp.router_bias, k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_or, p_or, margin, logits, k)


@pytest.mark.parametrize("T,D,E,k", [
    (64, 128, 8, 2), (300, 2880, 32, 4), (97, 7168, 256, 8), (33, 136, 17, 5), (70, 512, 128, 6)])
def test_router_parity_selection_bias(T, D, E, k):
    """Selection-only bias (load balancing): ids from logit + bias, weights from
    the plain logits, on both top-k paths (E <= 64 and E > 64)."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=8, router_bias=True, bias_select=True)
    inp = W.make_inputs(s, seed=T + E)
    g = _gpu(inp)
    ids, w = moe.moe_route(g.x, g.w_g, k, g.router_bias, bias_select=True)
    torch.cuda.synchronize()
    ids_or, p_or, margin, keys = _route_oracle(inp, k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_or, p_or, margin, keys, k)
    # the bias must have moved selections, or the test proves nothing
    ids_plain, _, _, _ = oracle.route(inp.x, inp.w_g, None, k)
    assert np.mean(np.sort(ids_plain, 1) != np.sort(ids_or, 1)) > 0.05


def test_router_exact_ties_on_grid_inputs():
    """Exact fp32 ties (grid inputs): the GPU must take the lower index, like the oracle."""
    s = W.Shape(T=500, D=64, E=16, k=4, F=8)
    inp = W.make_grid_inputs(s, seed=7)
    g = _gpu(inp)
    ids, w = moe.moe_route(g.x, g.w_g, s.k)
    torch.cuda.synchronize()
    ids_or, p_or, margin, logits = oracle.route(inp.x, inp.w_g, None, s.k)
    assert np.any(margin == 0)
    assert np.array_equal(ids.cpu().numpy(), ids_or)  # logits are exact, so order is too


@pytest.mark.parametrize("E,k", [(32, 4), (256, 8)])  # 256: two 16-token tiles per workgroup
def test_router_batch_invariance(E, k):
    s = W.Shape(T=64, D=2880, E=E, k=k, F=8)
    inp = W.make_inputs(s, seed=3)
    g = _gpu(inp)
    ids, w = moe.moe_route(g.x, g.w_g, s.k)
    for t in (0, 15, 16, 31, 32, 63):
        i1, w1 = moe.moe_route(g.x[t:t + 1].contiguous(), g.w_g, s.k)
        assert torch.equal(i1[0], ids[t]) and torch.equal(w1[0], w[t])


@pytest.mark.parametrize("T,D,E,k", [(4096, 4096, 8, 2), (300, 2880, 32, 4), (200, 7168, 64, 6)])
def test_routing_bitwise_the_same_on_every_path(T, D, E, k):
    """A token's ids and weights are bitwise the same whether it is routed
    alone or in a batch of up to 64 tokens (partial logits finished in the
    route-finish kernel) or in a larger batch (the full router kernel), through
    moe_forward or moe_route."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=16)
    inp = W.make_inputs(s, seed=E + k)
    g = _gpu(inp)

    def fwd(x):
        n = x.shape[0]
        ids = torch.empty((n, k), dtype=torch.int32, device=DEV)
        w = torch.empty((n, k), dtype=torch.float32, device=DEV)
        moe.moe_forward(x, g.w_g, g.w_gate_up, g.w_down, k, topk_ids=ids, topk_w=w)
        return ids, w

    ids_all, w_all = fwd(g.x)                    # T > 64: the full router
    ids_r, w_r = moe.moe_route(g.x, g.w_g, k)
    assert torch.equal(ids_all, ids_r) and torch.equal(w_all, w_r)
    for n in (1, 5, 64):                         # few tokens: partial logits
        for t0 in (0, 37, T - n):
            xs = g.x[t0:t0 + n].contiguous()
            ids_f, w_f = fwd(xs)
            ids_q, w_q = moe.moe_route(xs, g.w_g, k)
            assert torch.equal(ids_f, ids_all[t0:t0 + n]) and torch.equal(w_f, w_all[t0:t0 + n]), (n, t0)
            assert torch.equal(ids_q, ids_f) and torch.equal(w_q, w_f), (n, t0)


# ---------------------------------------------------------------------- align
@pytest.mark.parametrize("T,k,E,shared", [(64, 2, 8, 0), (1000, 4, 32, 0), (513, 8, 256, 513),
                                          (1, 4, 32, 0), (4096, 2, 8, 4096), (3, 1, 1, 0),
                                          # T*k = 1024, the last size of the one-workgroup
                                          # kernel, and 1025, the first of the per-group one
                                          (128, 8, 64, 0), (205, 5, 64, 0), (205, 5, 64, 205)])
def test_align_parity_random_ids(T, k, E, shared):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    shape = moe.make_shape(T, 64, E, 64, k, 64 if shared else 0)
    bm = moe.moe_block_m(shape)
    out = moe.moe_align(torch.from_numpy(ids).to(DEV), E, bm, shared)
    torch.cuda.synchronize()
    ref = oracle.align(ids, E, bm, shared=bool(shared))
    align_equal({k_: v.cpu().numpy() for k_, v in out.items()}, ref)


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_align_parity_block_sizes_and_skew(bm):
    T, k, E = 777, 2, 8
    rng = np.random.default_rng(bm)
    # Zipf-like loads with two empty experts
    p = np.array([0.5, 0.3, 0.1, 0.05, 0.03, 0.02, 0.0, 0.0])
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    out = moe.moe_align(torch.from_numpy(ids).to(DEV), E, bm, 0)
    ref = oracle.align(ids, E, bm)
    align_equal({k_: v.cpu().numpy() for k_, v in out.items()}, ref)


def test_align_all_to_one_expert():
    T, k, E = 300, 2, 8
    ids = np.tile(np.array([[6, 1]], np.int32), (T, 1))
    out = moe.moe_align(torch.from_numpy(ids).to(DEV), E, 128, 0)
    align_equal({k_: v.cpu().numpy() for k_, v in out.items()}, oracle.align(ids, E, 128))


# ------------------------------------------------------------- routed layer
@pytest.mark.parametrize("T,D,E,k,F,Fs", [(200, 256, 8, 2, 384, 0), (1, 128, 4, 2, 64, 0),
                                          (300, 192, 16, 4, 136, 64)])
def test_forward_routed_parity(T, D, E, k, F, Fs):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T)
    ids_or, p_or, _, _ = oracle.route(inp.x, inp.w_g, None, k)
    g = _gpu(inp)
    y = moe.moe_forward_routed(g.x, g.w_gate_up, g.w_down, torch.from_numpy(ids_or).to(DEV),
                               torch.from_numpy(p_or.astype(np.float32)).to(DEV), g.ws_gate_up,
                               g.ws_down)
    torch.cuda.synchronize()
    y_ref = oracle.experts(inp, ids_or, p_or.astype(np.float32).astype(np.float64))
    rel, _, _ = y_error(y.cpu().numpy(), y_ref)
    assert rel <= Y_TOL


# --------------------------------------------------------------- whole layer
LAYER_CASES = [
    # several tiles per expert and a ragged last tile in M, N and K
    (2048, 256, 8, 2, 512, 0, False),
    (1500, 320, 8, 2, 200, 0, False),
    (333, 2880, 32, 4, 2880, 0, False),
    (700, 512, 64, 8, 256, 256, False),
    (1024, 1024, 8, 2, 1024, 0, True),
    (5, 128, 8, 2, 256, 0, False),
    (64, 128, 8, 2, 256, 0, False),
    (24, 200, 8, 2, 136, 0, False),   # 16-row tiles with ragged K chunks in both GEMMs
]


@pytest.mark.parametrize("T,D,E,k,F,Fs,bias", LAYER_CASES)
def test_layer_parity(T, D, E, k, F, Fs, bias):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=bias)
    _layer_parity(W.make_inputs(s, seed=T + E))


@pytest.mark.parametrize("T,D,E,k,F,Fs", [
    (4096, 256, 8, 2, 4096, 0),      # every expert over several m-tiles, a ragged last one
    (3000, 320, 8, 2, 4000, 1000),   # ragged N and K; the shared expert's narrower N
])
def test_layer_many_gate_up_rounds(T, D, E, k, F, Fs):
    """Shapes with at least four rounds of 256 x 256 gate/up tiles (no tile cut
    over K), experts over several m-tiles with ragged last ones, ragged N and K
    and a shared expert narrower than the routed ones: every token against
    the oracle."""
    bm = moe.moe_block_m(moe.make_shape(T, D, E, F, k, Fs))
    assert bm == 256
    m_tiles_min = -(-T * k // 256) + (-(-T // 256) if Fs else 0)
    assert m_tiles_min * -(-max(F, Fs) // 128) >= 4 * 256
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    _layer_parity(W.make_inputs(s, seed=T + F))


def staged_decode_tiles(T, D, E, k, F, Fs):
    """Whether both forward GEMMs of a bf16 layer run the weight-staging
    16/32-row tiles: the decode tile family (BM < 256) with the wide column
    tiles, which the launcher takes when the host's bound on occupied row
    tiles times the column tiles (32 outputs for gate/up, 64 for down) is at
    least 512 workgroups."""
    bm = moe.moe_block_m(moe.make_shape(T, D, E, F, k, Fs))
    A = T * k
    busy = max(min(A, E), -(-A // bm)) + (-(-T // bm) if Fs else 0)
    return bm < 256 and busy * -(-max(F, Fs) // 32) >= 512 and busy * -(-D // 64) >= 512


def narrow_decode_tiles(T, D, E, k, F, Fs):
    """Whether both forward GEMMs take the narrow column tiles (16 outputs per
    workgroup, still staged through LDS for bf16): fewer than 512 workgroups
    with the wide ones."""
    bm = moe.moe_block_m(moe.make_shape(T, D, E, F, k, Fs))
    A = T * k
    busy = max(min(A, E), -(-A // bm)) + (-(-T // bm) if Fs else 0)
    return bm < 256 and busy * -(-max(F, Fs) // 32) < 512 and busy * -(-D // 64) < 512


STAGED_CASES = [
    (256, 1000, 64, 8, 1000, 136),  # 32-row tiles; N % 32 = 8, K % 64 = 40; shared expert
    (64, 1000, 32, 4, 1000, 0),     # 16-row tiles; the same ragged N and K
    (1024, 192, 256, 8, 136, 0),    # 32-row tiles; K = 192 and 136 leave waves without a chunk
]
NARROW_CASES = [
    (1, 1000, 32, 4, 1000, 0),      # one token: N % 16 = 8, K % 64 = 40
    (3, 200, 8, 2, 136, 64),        # shared expert; K = 200 and 136, N = 136 and 64
    (1, 2880, 32, 4, 2880, 0),      # the gpt-oss shape at one token
    (2, 512, 64, 8, 384, 0),        # top-8 of 64 experts
]


@pytest.mark.parametrize("T,D,E,k,F,Fs", NARROW_CASES)
def test_layer_narrow_decode_tiles_ragged(T, D, E, k, F, Fs):
    """The narrow staged decode tiles (32 and 16 weight rows per stage) on
    ragged shapes and a few tokens."""
    assert narrow_decode_tiles(T, D, E, k, F, Fs)
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    _layer_parity(W.make_inputs(s, seed=T + F))


@pytest.mark.parametrize("T,D,E,k,F,Fs", STAGED_CASES)
def test_layer_staged_decode_tiles_ragged(T, D, E, k, F, Fs):
    """The LDS-staged decode tiles on ragged shapes: weight rows past N
    masked, 8-wide K pieces past K masked, and waves with no K chunk."""
    assert staged_decode_tiles(T, D, E, k, F, Fs)
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    _layer_parity(W.make_inputs(s, seed=T + F))


@pytest.mark.parametrize("T,D,E,k,F,Fs", [
    (64, 2880, 32, 4, 512, 0),     # few tokens: partial logits, routing finished per token
    (7, 512, 64, 6, 256, 256),     # few tokens, 64 experts, shared expert
    (300, 1024, 8, 2, 512, 0),     # full router, E <= 64 top-k
    (40, 1024, 256, 8, 256, 256),  # full router, E > 64 top-k
])
def test_layer_selection_bias(T, D, E, k, F, Fs):
    """Whole layer with a selection-only router bias against the oracle."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=True, bias_select=True)
    _layer_parity(W.make_inputs(s, seed=T + E + 1))


@pytest.mark.parametrize("T", [16, 200])
def test_layer_selection_bias_forces_expert_not_weight(T):
    """+1000 on expert 3: it is every token's slot 0, with the weight the plain
    logits give it (a bias inside the logits would give it weight ~1)."""
    s = W.Shape(T=T, D=512, E=8, k=2, F=256, router_bias=True, bias_select=True)
    inp = W.make_inputs(s, seed=5)
    inp.router_bias = torch.zeros(8, dtype=torch.float32)
    inp.router_bias[3] = 1000.0
    _, ids, w = _layer_parity(inp)
    assert np.all(ids[:, 0] == 3)
    assert w[:, 0].min() < 0.5


@pytest.mark.parametrize("T,D,E,k,F,Fs,sel,shard", [
    (64, 2880, 32, 4, 256, 0, False, None),    # few tokens: routing finished in align
    (300, 512, 8, 2, 256, 128, True, None),    # shared expert: last entry is T
    (700, 512, 64, 8, 256, 0, False, (16, 40)),  # a shard: its held experts only
    (0, 256, 8, 2, 256, 0, False, None),       # no tokens: all zeros
])
def test_expert_load_counts(T, D, E, k, F, Fs, sel, shard):
    """moe_expert_load: bit-exact per-expert counts of the last call's routing."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=sel, bias_select=sel)
    g = _gpu(W.make_inputs(s, seed=T + 3))
    a, b = shard if shard else (0, E)
    gu, dn = g.w_gate_up[a:b].contiguous(), g.w_down[a:b].contiguous()
    eb = a if shard else None
    shape = moe.layer_shape(g.x, g.w_g, gu, k, g.ws_gate_up, g.router_bias, bias_select=sel,
                            expert_begin=eb)
    ws = moe.alloc_workspace(shape, DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    moe.moe_forward(g.x, g.w_g, gu, dn, k, g.router_bias, g.ws_gate_up, g.ws_down, topk_ids=ids,
                    workspace=ws, expert_begin=eb, bias_select=sel)
    G = (b - a) + (1 if Fs else 0)
    counts = torch.full((G,), -7, dtype=torch.int32, device=DEV)
    moe.moe_expert_load(shape, ws, counts)
    torch.cuda.synchronize()
    flat = ids.cpu().numpy().ravel()
    expect = np.bincount(flat[(flat >= a) & (flat < b)] - a, minlength=b - a)
    if Fs:
        expect = np.append(expect, T)
    assert np.array_equal(counts.cpu().numpy(), expect)


def test_expert_load_drives_selection_bias_balancing():
    """The loop the two pieces make: loads out of moe_expert_load, a
    selection-only bias nudged against the over-loaded experts, repeated;
    the most loaded expert's share must drop well below where it started."""
    s = W.Shape(T=1024, D=256, E=8, k=2, F=256, router_bias=True, bias_select=True)
    inp = W.make_inputs(s, seed=0)
    inp.x += 0.25       # a direction every token shares ...
    inp.w_g[0] += 0.02  # ... that expert 0 scores: it is in most tokens' top-2
    g = _gpu(inp)
    b = torch.zeros(8, dtype=torch.float32, device=DEV)
    shape = moe.layer_shape(g.x, g.w_g, g.w_gate_up, 2, None, b, bias_select=True)
    ws = moe.alloc_workspace(shape, DEV)
    shares = []
    for _ in range(12):
        moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, 2, b, workspace=ws, bias_select=True)
        load = moe.moe_expert_load(shape, ws).float()
        share = load / load.sum()
        shares.append(share.max().item())
        b -= 0.1 * torch.sign(share - 1.0 / 8)
    torch.cuda.synchronize()
    print("max expert share per step:", ["%.3f" % v for v in shares])
    assert shares[0] > 0.3
    assert min(shares[-4:]) < 0.6 * shares[0]


FP8_CASES = [
    (64, 2880, 32, 4, 2880, 0),   # gpt-oss-shaped decode, 16-row tiles
    (300, 512, 64, 8, 256, 256),  # 32-row tiles, shared expert
    (40, 200, 8, 2, 136, 0),      # K tails: D and F not multiples of 64 (nor of 16)
    (5, 128, 8, 2, 256, 64),
    (1, 1024, 16, 4, 512, 0),
    (2048, 256, 8, 2, 512, 0),    # 256-row tiles
    (1500, 320, 8, 2, 208, 0),    # 256-row tiles, ragged M, N and K (F % 64 == 16)
    (1500, 320, 8, 2, 200, 0),    # F % 16 == 8: E4M3 keeps the 32-row tiles at any T
    (700, 512, 16, 4, 256, 256),  # 256-row tiles with the shared expert
    (512, 512, 8, 2, 512, 0),     # both GEMMs cut along K in their last round
]


@pytest.mark.parametrize("T,D,E,k,F,Fs", FP8_CASES)
def test_layer_fp8_weights(T, D, E, k, F, Fs):
    """E4M3 expert weights with per-row scales against the oracle."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, fp8=True)
    bm = moe.moe_block_m(moe.make_shape(T, D, E, F, k, Fs, weight_format=1))
    print("BM =", bm)
    if F % 16 or D % 16:
        assert bm in (16, 32)
    elif T * k > 48 * E:
        assert bm == 256
    _layer_parity(W.make_inputs(s, seed=T + D))


@pytest.mark.parametrize("T,D,E,k,F,Fs", FP8_CASES[:4] + FP8_CASES[5:8])
def test_layer_fp8_power_of_two_scales_match_bf16(T, D, E, k, F, Fs):
    """With power-of-two row scales every dequantised weight is a bf16 value
    and the scaling commutes with every rounding, so the E4M3 kernels and the
    bf16 kernels on the dequantised weights compute the same sums; they group
    K differently (128- vs 64-wide chunks), so y may differ by fp32 summation
    order and the rare bf16 rounding of an h element that lands on the other
    side.  With scales up to 2^-7 a weight reaches 3.5, so one such h moves a
    y element by a fraction of a percent of RMS (emulated in
    tests/test_tolerances.py): bounded at KSPLIT_TOL, and the routing must
    agree bit for bit."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, fp8=True)
    inp = W.make_inputs(s, seed=T + 1)
    rng = np.random.default_rng(T)

    def p2(t):
        return torch.tensor(2.0 ** rng.integers(-12, -6, size=tuple(t.shape)), dtype=torch.float32)

    inp.w_gate_up_scale, inp.w_down_scale = p2(inp.w_gate_up_scale), p2(inp.w_down_scale)
    if Fs:
        inp.ws_gate_up_scale, inp.ws_down_scale = p2(inp.ws_gate_up_scale), p2(inp.ws_down_scale)

    def deq(q, sc):
        return (q.view(torch.float8_e4m3fn).to(torch.float32) * sc[..., None]).to(torch.bfloat16)

    bf = dataclasses.replace(inp, shape=dataclasses.replace(s, fp8=False),
                             w_gate_up=deq(inp.w_gate_up, inp.w_gate_up_scale),
                             w_down=deq(inp.w_down, inp.w_down_scale),
                             ws_gate_up=deq(inp.ws_gate_up, inp.ws_gate_up_scale) if Fs else None,
                             ws_down=deq(inp.ws_down, inp.ws_down_scale) if Fs else None,
                             w_gate_up_scale=None, w_down_scale=None, ws_gate_up_scale=None,
                             ws_down_scale=None)
    y8, ids8, w8 = _forward(inp)
    yb, idsb, wb = _forward(bf)
    assert np.array_equal(ids8, idsb) and np.array_equal(w8, wb)
    rel, _, _ = y_error(y8, yb.astype(np.float64))
    print("E4M3 vs bf16 kernels: max|dy|/RMS = %.3g" % rel)
    assert rel <= TL.KSPLIT_TOL


def test_layer_fp8_shard_and_routed():
    """E4M3 weights in an expert-parallel shard and under a given routing."""
    s = W.Shape(T=64, D=512, E=16, k=4, F=256, Fs=0, fp8=True)
    inp = W.make_inputs(s, seed=9)
    g = _gpu(inp)
    ids_or, p_or, _, _ = oracle.route(inp.x, inp.w_g, None, s.k)
    a, b = 4, 12
    sc = (g.w_gate_up_scale[a:b].contiguous(), g.w_down_scale[a:b].contiguous(), None, None)
    y = moe.moe_forward_routed(g.x, g.w_gate_up[a:b].contiguous(), g.w_down[a:b].contiguous(),
                               torch.from_numpy(ids_or).to(DEV),
                               torch.from_numpy(p_or.astype(np.float32)).to(DEV),
                               n_experts=s.E, expert_begin=a, scales=sc)
    torch.cuda.synchronize()
    sh = dataclasses.replace(inp, w_gate_up=inp.w_gate_up[a:b].contiguous(),
                             w_down=inp.w_down[a:b].contiguous(),
                             w_gate_up_scale=inp.w_gate_up_scale[a:b].contiguous(),
                             w_down_scale=inp.w_down_scale[a:b].contiguous())
    y_ref = oracle.experts(sh, ids_or, p_or.astype(np.float32).astype(np.float64), expert_begin=a,
                           n_local=b - a)
    rel, _, _ = y_error(y.cpu().numpy(), y_ref)
    assert rel <= Y_TOL


def _run_mtiles(counts):
    """256-row m-tiles that run: a group of two or more m-tiles whose last one
    would hold at most 32 rows folds them into the m-tile before it."""
    n = 0
    for c in counts:
        mg = (int(c) + 255) // 256
        n += mg - (1 if mg >= 2 and c - (mg - 1) * 256 <= 32 else 0)
    return n


def _split(V, ctas, kmin):
    """(R, S) of the prefill GEMMs' last-round split: R tiles cut in S pieces."""
    if V % ctas == 0 or V >= 4 * ctas:
        return 0, 1
    R = V % ctas
    S = min(8, ctas // R, ((kmin + 63) // 64) // 4)
    return (R, S) if S >= 2 else (0, 1)


@pytest.mark.parametrize("T,D,E,k,F,Fs", [
    (512, 512, 8, 2, 512, 0),      # both GEMMs split (S = 2 at even expert loads)
    (2048, 512, 8, 2, 2048, 0),    # down split up to eight ways
    (1024, 512, 8, 2, 1024, 512),  # shared expert with a shorter K in the down GEMM
    (600, 1024, 4, 1, 4096, 0),    # few tiles, long K
])
def test_layer_split_last_round(T, D, E, k, F, Fs):
    """Tiles of a partial last round are cut along K, and the last piece to
    arrive sums the partials: parity, bitwise repeatability, and that the
    split really ran for these shapes."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T + F)
    shape = moe.make_shape(T, D, E, F, k, Fs)
    assert moe.moe_block_m(shape) == 256
    y1, ids, _ = _layer_parity(inp)
    # again with a workspace full of 0xFF bytes: the fp32 partial tiles then
    # hold NaNs, so y is only equal if every piece writes its partial tile
    # before the fixup kernel reads it
    g = _gpu(inp)
    ws = moe.alloc_workspace(shape, DEV)
    ws.view(torch.uint8).fill_(0xFF)
    y2 = moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, k, None, g.ws_gate_up, g.ws_down,
                         workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2.cpu().numpy())
    counts = np.bincount(ids.ravel(), minlength=E)
    mt = _run_mtiles(list(counts) + ([T] if Fs else []))
    ctas = min(256, torch.cuda.get_device_properties(0).multi_processor_count)
    fmax = max(F, Fs)
    _, s_gu = _split(mt * ((fmax + 127) // 128), ctas, D)
    _, s_dn = _split(mt * ((D + 255) // 256), ctas, min(F, Fs) if Fs else F)
    if (T, F) == (2048, 2048) or (T, F) == (600, 4096):
        assert s_dn >= 2  # the down GEMM is the one cut for these shapes
    print("m-tiles %d: gate/up S=%d, down S=%d" % (mt, s_gu, s_dn))
    assert max(s_gu, s_dn) >= 2


def _shard_inputs(inp, a, b, with_shared):
    return W.LayerInputs(inp.shape if with_shared else dataclasses.replace(inp.shape, Fs=0), inp.x,
                         inp.w_g, inp.w_gate_up[a:b].contiguous(), inp.w_down[a:b].contiguous(),
                         inp.router_bias, inp.ws_gate_up if with_shared else None,
                         inp.ws_down if with_shared else None)


@pytest.mark.parametrize("T,D,E,k,F,Fs,bounds", [
    (300, 256, 8, 2, 384, 64, [0, 2, 4, 6, 8]),                  # 256-row tiles, shared on shard 0
    (64, 2880, 32, 4, 2880, 0, [0, 4, 8, 12, 16, 20, 24, 28, 32]),  # gpt-oss decode over 8 shards
    (2048, 512, 8, 2, 1024, 0, [0, 3, 8]),                        # uneven shards, K-split tail
    (5, 128, 8, 2, 256, 0, [0, 1, 7, 8]),                         # shards that get no token
    (700, 512, 64, 8, 256, 256, [0, 16, 48, 64]),                 # 64 experts, top-8, shared
])
def test_layer_expert_shards(T, D, E, k, F, Fs, bounds):
    """Expert-parallel shards: each call holds a slice of the experts; its y
    matches the oracle's shard under the same routing, every shard routes
    identically, and the shards' y add up to the whole layer's."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T + 3 * E)
    g = _gpu(inp)
    y_full, ids_full, w_full = _forward(inp)
    ids_or, p_or, margin, logits = oracle.route(inp.x, inp.w_g, None, k)
    check_routing(ids_full, w_full, ids_or, p_or, margin, logits, k)
    y_or = oracle.experts(inp, ids_full, w_full.astype(np.float64))
    rms = float(np.sqrt(np.mean(np.square(y_or))))
    total = np.zeros_like(y_full, dtype=np.float64)
    for r, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        sh = r == 0
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        y = moe.moe_forward(g.x, g.w_g, g.w_gate_up[a:b].contiguous(), g.w_down[a:b].contiguous(), k,
                            None, g.ws_gate_up if sh else None, g.ws_down if sh else None,
                            topk_ids=ids, topk_w=w, expert_begin=a)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ids_full) and np.array_equal(w.cpu().numpy(), w_full)
        ref = oracle.experts(_shard_inputs(inp, a, b, sh), ids_full, w_full.astype(np.float64),
                             expert_begin=a, n_local=b - a)
        err = float(np.max(np.abs(y.cpu().numpy().astype(np.float64) - ref)))
        print("shard %d [%d, %d): max|err|/RMS(layer) = %.4g" % (r, a, b, err / rms))
        assert err <= Y_TOL * rms
        total += y.cpu().numpy()
    # not bitwise: a shard's tile count changes the K-split of its GEMMs, and a
    # different fp32 summation order can move h by one bf16 ulp; the bar is
    # derived from the count of such flips in tests/test_tolerances.py
    assert float(np.max(np.abs(total - y_full))) <= TL.SHARD_SUM_TOL * rms


def test_layer_E1_k1_dense_ffn():
    s = W.Shape(T=100, D=256, E=1, k=1, F=512)
    y, ids, w = _layer_parity(W.make_inputs(s, seed=1))
    assert np.all(ids == 0) and np.all(w == 1.0)


def test_layer_k_equals_E():
    s = W.Shape(T=100, D=128, E=4, k=4, F=128)
    _layer_parity(W.make_inputs(s, seed=2))


def test_layer_all_tokens_to_one_expert_and_empty_experts():
    """A +100 bias on one expert sends every token there first; others stay empty."""
    s = W.Shape(T=400, D=256, E=8, k=1, F=256, router_bias=True)
    inp = W.make_inputs(s, seed=4)
    inp.router_bias = torch.tensor([-100, -100, -100, 100, -100, -100, -100, -100], dtype=torch.float32)
    y, ids, w = _layer_parity(inp)
    assert np.all(ids == 3)


def test_layer_zero_tokens():
    s = W.Shape(T=0, D=128, E=8, k=2, F=256)
    inp = W.make_inputs(s, seed=0)
    y, ids, w = _forward(inp)
    assert y.shape == (0, 128)


def test_layer_deterministic_and_scaling():
    s = W.Shape(T=777, D=512, E=16, k=4, F=384, Fs=128)
    inp = W.make_inputs(s, seed=9)
    y1, i1, w1 = _forward(inp)
    y2, i2, w2 = _forward(inp)
    assert np.array_equal(y1, y2) and np.array_equal(i1, i2) and np.array_equal(w1, w2)
    inp2 = W.LayerInputs(s, inp.x, inp.w_g, inp.w_gate_up, (inp.w_down * 2).contiguous(), None,
                         inp.ws_gate_up, (inp.ws_down * 2).contiguous())
    y3, _, _ = _forward(inp2)
    assert np.array_equal(y3, 2 * y1)  # power-of-two scaling commutes with every rounding


def test_layer_poisoned_workspace_and_guards():
    """A NaN-filled workspace must not leak into y (padding rows are never read),
    and bytes around y stay untouched."""
    s = W.Shape(T=300, D=256, E=8, k=2, F=320, Fs=64)
    inp = W.make_inputs(s, seed=10)
    g = _gpu(inp)
    shape = moe.make_shape(300, 256, 8, 320, 2, 64)
    ws = moe.alloc_workspace(shape, DEV)
    ws.view(torch.uint8).fill_(0xFF)  # every float in it is NaN
    y_ref = moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, 2, None, g.ws_gate_up, g.ws_down)
    guard = torch.full((300 * 256 + 2 * 64,), 12345.0, dtype=torch.float32, device=DEV)
    y = guard[64:64 + 300 * 256].view(300, 256)
    moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, 2, None, g.ws_gate_up, g.ws_down, y=y,
                    workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.all(guard[:64] == 12345.0) and torch.all(guard[-64:] == 12345.0)


def test_errors_are_raised_before_launch():
    s = W.Shape(T=16, D=128, E=8, k=2, F=256)
    g = _gpu(W.make_inputs(s, seed=0))
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, 2, workspace=small)
    assert ei.value.code == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, 9)
    assert ei.value.code in (moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED)


# Group sizes whose last 256-row m-tile would hold at most 32 rows fold those
# rows into the m-tile before it: 270 and 288 (two m-tiles, 14 and 32 rows
# folded), 513, 1030 and 1056 (three to five m-tiles, 1, 6 and 32 folded);
# 289 and 650 do not fold (33 and 138 rows left), 20 is one tile.  Their sum,
# 4116 = 16 * 256 + 20, makes the shared expert's last 20 rows fold too.
FOLDED = [270, 288, 289, 513, 1030, 1056, 650, 20]


@pytest.mark.parametrize("counts,D,F,fp8", [
    ([257, 300, 511, 512, 256, 1, 0, 700], 256, 320, False),
    # one-tile groups at the row tiers' edges (64-row steps pick the A loads per
    # stage) and at 32-row sub-tile edges
    ([64, 65, 192, 193, 33, 32, 128, 129], 256, 320, False),
    # folded rows, with K and N tails in both GEMMs (136 = 2 * 64 + 8, 200 = 3 * 64 + 8)
    (FOLDED, 136, 200, False),
    (FOLDED, 256, 320, False),
    (FOLDED, 256, 320, True),
])
def test_forward_routed_tile_boundaries(counts, D, F, fp8):
    """256-row tiles at group sizes around tile boundaries (k = 1, so the counts are
    exact): 257, 300, 511 and 700 rows (two- and three-m-tile groups; 257 folds its
    last row into the first m-tile, the other two-tile ones split evenly), 512 and 256
    (full tiles), 1 row and an empty expert; one-tile groups on both sides of 32, 64,
    128 and 192 rows; the folded-row sizes above, with bf16 and E4M3 weights; tokens
    in shuffled order so every tile gathers scattered rows."""
    T = sum(counts)
    assert moe.moe_block_m(moe.make_shape(T, D, len(counts), F, 1, weight_format=int(fp8))) == 256
    s = W.Shape(T=T, D=D, E=len(counts), k=1, F=F, Fs=64, fp8=fp8)
    inp = W.make_inputs(s, seed=11)
    order = np.random.default_rng(5).permutation(T)
    ids = np.repeat(np.arange(len(counts)), counts)[order].astype(np.int32).reshape(T, 1)
    p = np.ones((T, 1), np.float32)
    g = _gpu(inp)
    y = moe.moe_forward_routed(g.x, g.w_gate_up, g.w_down, torch.from_numpy(ids).to(DEV),
                               torch.from_numpy(p).to(DEV), g.ws_gate_up, g.ws_down,
                               scales=_scales(g))
    torch.cuda.synchronize()
    y_ref = oracle.experts(inp, ids, p.astype(np.float64))
    rel, _, _ = y_error(y.cpu().numpy(), y_ref)
    print("counts %s D=%d F=%d fp8=%s: max|err|/RMS=%.4g" % (counts, D, F, fp8, rel))
    assert rel <= Y_TOL


def test_folded_rows_are_bitwise_the_rows_of_a_tile():
    """A row's arithmetic does not depend on which tile computes it: with 1030
    and 270 rows (6 and 14 rows folded into the tile before, computed by the
    written-out MFMAs) every token's y is bitwise the y of a call that holds
    only the unfolded tokens (groups of 1024 and 256 rows, no folding) or the
    folded ones with 100 others of each expert (one-tile groups of 106 and 114
    rows, still 256-row tiles: T k > 48 E)."""
    counts = [1030, 270]
    T, D, F = sum(counts), 256, 320
    s = W.Shape(T=T, D=D, E=2, k=1, F=F, Fs=0)
    inp = W.make_inputs(s, seed=21)
    ids = np.repeat(np.arange(2), counts).astype(np.int32).reshape(T, 1)
    p = np.ones((T, 1), np.float32)
    g = _gpu(inp)

    def run(tok):
        return moe.moe_forward_routed(g.x[tok].contiguous(), g.w_gate_up, g.w_down,
                                      torch.from_numpy(ids[tok]).to(DEV),
                                      torch.from_numpy(p[tok]).to(DEV))

    y = run(np.arange(T))
    keep = np.r_[0:1024, 1030:1030 + 256]       # rows of the 256-row tiles
    folded = np.r_[1024:1030, 1030 + 256:T]     # the folded rows
    mixed = np.r_[0:100, 1024:1030, 1030:1130, 1030 + 256:T]
    assert moe.moe_block_m(moe.make_shape(mixed.size, D, 2, F, 1)) == 256
    y_keep, y_mixed = run(keep), run(mixed)
    torch.cuda.synchronize()
    assert torch.equal(y[keep], y_keep)
    assert torch.equal(y[folded], y_mixed[torch.from_numpy(np.isin(mixed, folded)).to(DEV)])
    y_ref = oracle.experts(inp, ids, p.astype(np.float64))
    rel, _, _ = y_error(y.cpu().numpy(), y_ref)
    assert rel <= Y_TOL


def test_folded_rows_in_split_tiles():
    """Folded rows in tiles cut along K (a short last round: every tile is cut
    into two pieces here, K = 520 is nine stages): parity, and bitwise the same
    y from a workspace full of NaN bytes."""
    counts = [270, 1030, 20, 513]
    T, D, F = sum(counts), 520, 520
    s = W.Shape(T=T, D=D, E=len(counts), k=1, F=F, Fs=0)
    inp = W.make_inputs(s, seed=23)
    order = np.random.default_rng(7).permutation(T)
    ids = np.repeat(np.arange(len(counts)), counts)[order].astype(np.int32).reshape(T, 1)
    p = np.ones((T, 1), np.float32)
    g = _gpu(inp)
    ctas = min(256, torch.cuda.get_device_properties(0).multi_processor_count)
    mt = _run_mtiles(counts)
    assert _split(mt * ((F + 127) // 128), ctas, D)[1] >= 2
    assert _split(mt * ((D + 255) // 256), ctas, F)[1] >= 2
    shape = moe.make_shape(T, D, len(counts), F, 1)
    outs = []
    for fill in (None, 0xFF):
        ws = moe.alloc_workspace(shape, DEV)
        if fill is not None:
            ws.view(torch.uint8).fill_(fill)
        outs.append(moe.moe_forward_routed(g.x, g.w_gate_up, g.w_down, torch.from_numpy(ids).to(DEV),
                                           torch.from_numpy(p).to(DEV), workspace=ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    y_ref = oracle.experts(inp, ids, p.astype(np.float64))
    rel, _, _ = y_error(outs[0].cpu().numpy(), y_ref)
    print("folded rows in split tiles: max|err|/RMS=%.4g" % rel)
    assert rel <= Y_TOL
