"""Derivations of the GPU tests' parity bars, on the CPU.

Each bar in tests/tolerances.py is set from an emulation of the roundings the
GPU path takes (bf16 storage of h and of the gradients' GEMM operands, fp32
accumulation in K chunks, the K-split of a GEMM's last round), run on the
shapes the GPU tests use and compared with the oracle or with itself.  Each
test asserts that the bar sits a stated factor above the largest emulated
error, and, where a bar also has to catch mistakes, that planted mistakes
exceed it.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import tolerances as TL

TAG_DY = 99  # the dy stream of the backward GPU tests


def _rel_max(a, b, rms):
    return float(np.max(np.abs(a - b))) / rms


# ------------------------------------------------------------------ forward y
# (T, D, E, k, F, Fs, elements of y at the workload's full size).  The
# Mixtral- and DeepSeek-shaped rows keep the width, the expert size and k of
# their workloads with fewer tokens and experts: the error of one y element
# depends on D, F and the routing weights, not on how many experts there are.
FWD_CASES = [
    (64, 128, 8, 2, 256, 0, 64 * 128),
    (16, 4096, 2, 2, 14336, 0, 4096 * 4096),
    (64, 2880, 32, 4, 2880, 0, 64 * 2880),
    (8, 7168, 16, 8, 2048, 2048, 8192 * 7168),
]


@pytest.mark.parametrize("T,D,E,k,F,Fs,n_full", FWD_CASES)
def test_forward_bar_is_twice_the_h_rounding(T, D, E, k, F, Fs, n_full):
    """The GPU stores h = SiLU(g) u in bf16 between the gate/up and down GEMMs;
    the oracle keeps it exact.  That rounding (relative 2^-9 at most per h)
    summed over F terms of random sign gives every y element a Gaussian error
    of about 0.17% of RMS(y); the largest of N elements sits near
    sqrt(2 ln N) of those, 0.8-1.0% of RMS at the workloads' full sizes.
    Y_TOL = 2% leaves a factor 2 above it, while a lost, doubled or
    mis-weighted expert output moves y by tens of percent (planted below)."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T + 1)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, None, k)
    y0 = oracle.experts(inp, ids, p)
    y, _ = TL.emulate_forward(inp, ids, p)
    rms = float(np.sqrt(np.mean(y0 * y0)))
    d = (y - y0) / rms
    e_rms = float(np.sqrt(np.mean(d * d)))
    kurt = float(np.mean(d ** 4)) / e_rms ** 4
    full = e_rms * np.sqrt(2 * np.log(n_full))
    print("h rounding: max %.4g, RMS %.4g, kurtosis %.2f, expected max at full size %.4g (of RMS)"
          % (np.max(np.abs(d)), e_rms, kurt, full))
    assert kurt < 3.5  # Gaussian: the extreme-value estimate applies
    assert 1e-3 < e_rms < 2.5e-3
    assert np.max(np.abs(d)) <= TL.Y_TOL / 1.8 and full <= TL.Y_TOL / 1.8


@pytest.mark.parametrize("mistake", ["swap_gate_up", "slot_weights", "drop_slot"])
def test_forward_bar_catches_mistakes(mistake):
    s = W.Shape(T=64, D=128, E=8, k=2, F=256)
    inp = W.make_inputs(s, seed=65)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, None, s.k)
    y0 = oracle.experts(inp, ids, p)
    rms = float(np.sqrt(np.mean(y0 * y0)))
    if mistake == "swap_gate_up":  # SiLU applied to the up half
        wgu = lambda e: np.roll(TL.f64(inp.w_gate_up[e]), s.F, axis=0)  # noqa: E731
        y, _ = TL.emulate_forward(inp, ids, p, w_gate_up=wgu)
    elif mistake == "slot_weights":  # each token's weights given to the other slot
        y, _ = TL.emulate_forward(inp, ids, p[:, ::-1].copy())
    else:  # the second slot of the last token lost
        p2 = p.copy()
        p2[-1, 1] = 0.0
        y, _ = TL.emulate_forward(inp, ids, p2)
    err = _rel_max(y, y0, rms)
    print("%s: max|dy|/RMS = %.3g" % (mistake, err))
    assert err > 5 * TL.Y_TOL


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("D,E,k", [(4096, 8, 2), (2880, 32, 4), (7168, 256, 8), (128, 8, 2)])
def test_routing_margin_and_weight_bars(D, E, k):
    """The GPU's logits are fp32 sums of bf16 products taken in K chunks (one
    wave's chunks, then the waves' partial sums); the oracle's are exact sums
    rounded once to fp32.  Emulated over 256 tokens in two orders, the two
    differ by at most ~6e-6 (D = 7168).  A top-k choice can only differ where
    the k-th and (k+1)-th logits are closer than twice that, so MARGIN = 1e-4
    covers it with a factor 8.  The routing weights are a softmax over the
    chosen logits, whose Jacobian rows sum to 2 p (1 - p) <= 1/2 in absolute
    value, so they move by at most half the logit error, plus a few fp32 ulps
    of the GPU's exp and division: far inside WEIGHT_TOL = 1e-4."""
    s = W.Shape(T=256, D=D, E=E, k=k, F=8)
    inp = W.make_inputs(s, seed=5)
    ids, p, margin, lg = oracle.route(inp.x, inp.w_g, None, k)
    x, wg = TL.f64(inp.x), TL.f64(inp.w_g)
    dl = 0.0
    for pieces, chunk in ((1, 16), (16, 16), (4, 32)):
        em = TL.fp32_dot(x, wg, pieces, chunk)
        dl = max(dl, float(np.max(np.abs(em - lg))))
        # weights from the emulated logits where the choice agrees
        sel = np.take_along_axis(em, ids.astype(np.int64), 1)
        q = np.exp(sel - sel.max(1, keepdims=True))
        q /= q.sum(1, keepdims=True)
        assert np.max(np.abs(q - p)) <= 0.5 * dl + 1e-12
    near = int(np.sum(margin <= TL.MARGIN))
    print("max|logit error| %.3g; %d of 256 tokens within MARGIN of a tie" % (dl, near))
    assert 2 * dl <= TL.MARGIN / 8
    assert 0.5 * dl + 8 * 2.0 ** -24 <= TL.WEIGHT_TOL / 10


# ------------------------------------------------------------------ shard sums
# The expert-parallel shard test's shapes and the K-splits emulated; the
# gpt-oss-shaped row holds 8 experts instead of 32 (the flips depend on D, F
# and the order of the sums, not on how many experts there are).
SHARD_CASES = [
    (300, 256, 8, 2, 384, 64, (2, 4, 8)),
    (64, 2880, 8, 4, 2880, 0, (2, 8)),
    (2048, 512, 8, 2, 1024, 0, (2, 4, 8)),
    (700, 512, 64, 8, 256, 256, (2, 4, 8)),
]


@pytest.mark.parametrize("T,D,E,k,F,Fs,splits", SHARD_CASES)
def test_shard_sum_bar_from_h_flips(T, D, E, k, F, Fs, splits):
    """A shard holds fewer experts, so fewer tiles, and its gate/up GEMM may
    cut K of its last round into S pieces where the whole layer does not (or
    the other way round).  The fp32 g and u then differ in their last bits,
    and where SiLU(g) u lies near a bf16 rounding boundary h lands one ulp
    apart.  Emulated with S = 2..8 against S = 1, 1e-4 to 4e-4 of the h
    elements flip and no token has more than 5 flips.  Each flip moves y by at
    most p |dh| max_d |W_down[d, f]|; summed over a token's flips this bounds
    the change of the shards' sum at 0.34% of RMS(y) on these shapes (the
    emulated change equals the bound: one flip dominates).  SHARD_SUM_TOL = 1%
    is three times the largest bound."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs)
    inp = W.make_inputs(s, seed=T + 3 * E)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, None, k)
    y1, h1 = TL.emulate_forward(inp, ids, p, pieces=1)
    rms = float(np.sqrt(np.mean(y1 * y1)))
    colmax = [np.abs(TL.f64(inp.w_down[e])).max(0) for e in range(E)]
    if Fs:
        colmax.append(np.abs(TL.f64(inp.ws_down)).max(0))
    for S in splits:
        y2, h2 = TL.emulate_forward(inp, ids, p, pieces=S)
        bound = np.zeros(T)
        flips = total = most = 0
        for e, (ts, a) in h1.items():
            b = h2[e][1]
            pw = np.ones(T) if e == E else p[ts, np.nonzero(ids == e)[1]]
            np.add.at(bound, ts, pw * (np.abs(a - b) @ colmax[e]))
            flips += int(np.sum(a != b))
            total += a.size
            most = max(most, int((a != b).sum(1).max()))
        dy = _rel_max(y1, y2, rms)
        bnd = float(bound.max()) / rms
        print("S=%d: %d of %d h flipped (%.2e), at most %d per token; max|dy| %.4g, flip bound %.4g"
              % (S, flips, total, flips / total, most, dy, bnd))
        assert 0 < flips <= 1e-3 * total and most <= 8
        assert dy <= bnd * (1 + 1e-6) + 1e-12
        assert bnd <= TL.SHARD_SUM_TOL / 2.5


# ------------------------------------------------------- E4M3 vs bf16 kernels
@pytest.mark.parametrize("T,D,E,k,F,Fs", [  # the GPU test's shapes (gpt-oss-shaped: 8 experts)
    (64, 2880, 8, 4, 2880, 0), (300, 512, 64, 8, 256, 256), (40, 200, 8, 2, 136, 0),
    (2048, 256, 8, 2, 512, 0), (512, 512, 8, 2, 512, 0),
])
def test_ksplit_bar_for_e4m3_against_bf16(T, D, E, k, F, Fs):
    """With power-of-two row scales the E4M3 kernels and the bf16 kernels on
    the dequantised weights compute the same products and group them into
    fp32 chunks of 128 and 64 along K.  Emulating both groupings on the GPU
    test's weights (scales 2^-12..2^-7, so weights up to 3.5) moves y by at
    most 0.22% of RMS (the gpt-oss-shaped case), under a quarter of
    KSPLIT_TOL."""
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, fp8=True)
    inp = W.make_inputs(s, seed=T + 1)
    rng = np.random.default_rng(T)

    def p2(t):
        return torch.tensor(2.0 ** rng.integers(-12, -6, size=tuple(t.shape)), dtype=torch.float32)

    gsc, dsc = p2(inp.w_gate_up_scale), p2(inp.w_down_scale)
    if Fs:
        sgsc, sdsc = p2(inp.ws_gate_up_scale), p2(inp.ws_down_scale)

    def deq(q, sc):
        return (q.view(torch.float8_e4m3fn).to(torch.float32) * sc[..., None]).to(torch.bfloat16)

    bf = dataclasses.replace(inp, shape=dataclasses.replace(s, fp8=False),
                             w_gate_up=deq(inp.w_gate_up, gsc), w_down=deq(inp.w_down, dsc),
                             ws_gate_up=deq(inp.ws_gate_up, sgsc) if Fs else None,
                             ws_down=deq(inp.ws_down, sdsc) if Fs else None,
                             w_gate_up_scale=None, w_down_scale=None, ws_gate_up_scale=None,
                             ws_down_scale=None)
    ids, p, _, _ = oracle.route(bf.x, bf.w_g, None, k)
    ya, _ = TL.emulate_forward(bf, ids, p, pieces=1, chunk=64)
    yb, _ = TL.emulate_forward(bf, ids, p, pieces=1, chunk=128)
    err = _rel_max(ya, yb, float(np.sqrt(np.mean(ya * ya))))
    print("chunks of 64 vs 128: max|dy|/RMS = %.3g" % err)
    assert err <= TL.KSPLIT_TOL / 4


# ------------------------------------------------------------------ gradients
BWD_CASES = [  # the backward GPU tests' shapes and seeds
    (64, 128, 8, 2, 256, 0, False), (300, 512, 64, 8, 256, 256, False),
    (40, 200, 8, 2, 136, 0, True), (2048, 256, 8, 2, 512, 0, False),
    (1500, 320, 8, 2, 200, 0, True), (700, 512, 16, 4, 256, 256, False),
    (32, 1024, 8, 2, 768, 256, False), (200, 1024, 16, 2, 640, 0, True),
    (200, 200, 16, 2, 136, 64, False), (64, 2048, 16, 2, 1024, 0, False),
    (64, 1000, 32, 4, 1000, 0, False), (256, 1000, 64, 8, 1000, 136, False),
]


def _backward_case(T, D, E, k, F, Fs, bias):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, router_bias=bias)
    inp = W.make_inputs(s, seed=T + F)
    ids, p, _, _ = oracle.route(inp.x, inp.w_g, inp.router_bias, k)
    p = p.astype(np.float32).astype(np.float64)
    dy = W.normal_f32((T, D), T, TAG_DY, 1.0).numpy()
    return inp, ids, p, dy, oracle.backward(inp, ids, p, dy)


def _grad_errors(got, ref, ids, p, E, bias):
    out = {}
    for name in ref:
        if name == "dp" or (name == "d_bias" and not bias):
            continue
        sc = TL.bias_terms_scale(ref["dp"], ids, p, E) if name == "d_bias" else 0.0
        out[name] = TL.grad_error(got[name], ref[name], sc)
    return out


@pytest.mark.parametrize("T,D,E,k,F,Fs,bias", BWD_CASES)
def test_gradient_bars_cover_bf16_operands(T, D, E, k, F, Fs, bias):
    """The gradient GEMMs take bf16 operands (dy, h, dg, du; x and the
    weights are bf16 already) and accumulate in fp32, whose error is 2^16
    times smaller.  The bf16 roundings put a relative error of up to 2^-9 on
    each product term: 0.2-0.3% of RMS on every gradient, and up to 9% of RMS
    on the largest entries of dW_down, whose rows are sums over as few as one
    routed token with heavy-tailed values (11.4% on the case with 8 rows per
    expert).  GRAD_RMS_TOL = 1% is 3 times the largest emulated RMS error and
    GRAD_MAX_TOL = 15% is 1.3 times the largest emulated entry error; the
    inputs are seeded, so the GPU sees exactly these roundings."""
    inp, ids, p, dy, ref = _backward_case(T, D, E, k, F, Fs, bias)
    em = TL.emulate_backward(inp, ids, p, dy)
    for name, (r, m) in _grad_errors(em, ref, ids, p, E, bias).items():
        print("%s: RMS err %.3g, max err %.3g (of RMS)" % (name, r, m))
        assert r <= TL.GRAD_RMS_TOL / 3 and m <= TL.GRAD_MAX_TOL / 1.3, name


@pytest.mark.parametrize("mistake", ["dsilu", "dl_sign", "dw_down_p"])
def test_gradient_bars_catch_mistakes(mistake):
    hit = []
    for case in [(64, 128, 8, 2, 256, 0, False), (40, 200, 8, 2, 136, 0, True)]:
        inp, ids, p, dy, ref = _backward_case(*case)
        em = TL.emulate_backward(inp, ids, p, dy, mistake=mistake)
        errs = _grad_errors(em, ref, ids, p, case[2], case[6])
        hit += [n for n, (r, m) in errs.items() if r > TL.GRAD_RMS_TOL or m > TL.GRAD_MAX_TOL]
    print("%s fails the bars on %s" % (mistake, sorted(set(hit))))
    assert hit
