"""Pins of the oracle's quantised expert weights (E4M3 codes, one fp32 scale per row).

"Mixture of Experts optimiza Transformers y LLMs" (section on the resources the
method needs) and "Transformers v5 El Secreto Detrás de los Modelos MoE Más
Rápidos" (section on its limits) name per-expert quantisation of the expert
weights without fixing a format.  Reading taken: OCP FP8 E4M3 codes with one
fp32 scale per weight row (per output channel) of every expert matrix, the
weight being code value times scale; activations stay bf16.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.dense_ref import dense_forward


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(mine[nan]))
    assert np.array_equal(mine[~nan], ref[~nan])


def test_decode_closed_forms():
    v = oracle.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x80, 0xB8, 0x40, 0x3C], np.uint8))
    assert list(v) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, 0.0, -1.0, 2.0, 1.5]
    assert np.signbit(v[5])


def _fp8_inputs(T, D, E, k, F, Fs=0, seed=0):
    s = W.Shape(T=T, D=D, E=E, k=k, F=F, Fs=Fs, fp8=True)
    return W.make_inputs(s, seed=seed)


def test_power_of_two_scales_equal_bf16_weights_bitwise():
    """With power-of-two scales (a different one per row) every dequantised
    weight is exactly a bf16 value, so the fp8 layer must equal, bit for bit,
    the bf16 layer on those values: this pins the row a scale belongs to."""
    inp = _fp8_inputs(24, 64, 4, 2, 32, Fs=16, seed=3)
    rng = np.random.default_rng(0)

    def p2(n):
        return torch.tensor(2.0 ** rng.integers(-12, -4, size=n), dtype=torch.float32)

    inp.w_gate_up_scale = p2(inp.w_gate_up_scale.shape).reshape(inp.w_gate_up_scale.shape)
    inp.w_down_scale = p2(inp.w_down_scale.shape).reshape(inp.w_down_scale.shape)
    inp.ws_gate_up_scale = p2(inp.ws_gate_up_scale.shape)
    inp.ws_down_scale = p2(inp.ws_down_scale.shape)

    def deq(q, sc):
        v = q.view(torch.float8_e4m3fn).to(torch.float32) * sc[..., None]
        b = v.to(torch.bfloat16)
        assert torch.equal(b.to(torch.float32), v)  # exact in bf16
        return b

    bf = dataclasses.replace(inp, shape=dataclasses.replace(inp.shape, fp8=False),
                             w_gate_up=deq(inp.w_gate_up, inp.w_gate_up_scale),
                             w_down=deq(inp.w_down, inp.w_down_scale),
                             ws_gate_up=deq(inp.ws_gate_up, inp.ws_gate_up_scale),
                             ws_down=deq(inp.ws_down, inp.ws_down_scale),
                             w_gate_up_scale=None, w_down_scale=None, ws_gate_up_scale=None,
                             ws_down_scale=None)
    y8, ids, p, _ = oracle.forward(inp)
    yb, ids_b, p_b, _ = oracle.forward(bf)
    assert np.array_equal(ids, ids_b) and np.array_equal(y8, yb)


@pytest.mark.parametrize("T,D,E,k,F,Fs", [(40, 64, 8, 2, 48, 0), (17, 128, 16, 4, 32, 24), (9, 32, 3, 3, 16, 8)])
def test_layer_matches_dense_with_library_decode(T, D, E, k, F, Fs):
    """General per-row scales: against the dense float64 evaluation, which
    decodes the codes with torch's float8_e4m3fn type."""
    inp = _fp8_inputs(T, D, E, k, F, Fs, seed=T)
    y, ids, p, margin = oracle.forward(inp)
    y_d, ids_d, _ = dense_forward(inp)
    assert np.all(margin > 1e-6)
    assert np.array_equal(ids, ids_d)
    assert np.max(np.abs(y - y_d)) < 1e-12 * max(1.0, np.abs(y_d).max())


def test_scale_is_linear_per_expert():
    """Doubling every scale of the down matrices doubles the routed output exactly."""
    inp = _fp8_inputs(32, 64, 8, 2, 32, seed=5)
    y1, _, _, _ = oracle.forward(inp)
    inp2 = dataclasses.replace(inp, w_down_scale=inp.w_down_scale * 2)
    y2, _, _, _ = oracle.forward(inp2)
    assert np.array_equal(y2, 2 * y1)


def test_quantiser_error_bound():
    """The inputs' quantiser: each dequantised weight is within half an E4M3
    step of the bf16 draw (relative 2^-4 for normals, plus the subnormal step)."""
    inp = W.make_inputs(W.Shape(T=4, D=256, E=4, k=2, F=128), seed=1)
    q, sc = W.quantize_rows_e4m3(inp.w_gate_up)
    deq = q.view(torch.float8_e4m3fn).to(torch.float64) * sc.double()[..., None]
    w = inp.w_gate_up.double()
    tol = np.abs(w.numpy()) * 2.0 ** -4 + 2.0 ** -10 * sc.double().numpy()[..., None] + 1e-30
    assert np.all(np.abs(deq.numpy() - w.numpy()) <= tol)
    # each row's largest magnitude maps to the top code 448
    assert torch.all(q.view(torch.float8_e4m3fn).float().abs().amax(-1) == 448.0)


def test_shard_sums_with_fp8():
    inp = _fp8_inputs(48, 64, 8, 2, 32, Fs=16, seed=7)
    y, ids, p, _ = oracle.forward(inp)
    acc = np.zeros_like(y)
    for a, b in [(0, 3), (3, 8)]:
        sh = dataclasses.replace(inp, w_gate_up=inp.w_gate_up[a:b].contiguous(),
                                 w_down=inp.w_down[a:b].contiguous(),
                                 w_gate_up_scale=inp.w_gate_up_scale[a:b].contiguous(),
                                 w_down_scale=inp.w_down_scale[a:b].contiguous())
        if a:
            sh = dataclasses.replace(sh, shape=dataclasses.replace(sh.shape, Fs=0), ws_gate_up=None,
                                     ws_down=None, ws_gate_up_scale=None, ws_down_scale=None)
        acc += oracle.experts(sh, ids, p, expert_begin=a, n_local=b - a)
    assert np.max(np.abs(acc - y)) < 1e-12 * np.abs(y).max()


def test_missing_scales_rejected():
    inp = _fp8_inputs(8, 32, 4, 2, 16, seed=1)
    bad = dataclasses.replace(inp, w_down_scale=None)
    with pytest.raises(ValueError):
        oracle.experts(bad, np.zeros((8, 2), np.int32) + np.array([0, 1], np.int32), np.full((8, 2), 0.5))
