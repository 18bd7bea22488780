"""Seeded synthetic workloads for one sparse-MoE SwiGLU feed-forward layer.

This module only *draws inputs* and counts sizes.  It contains none of the
layer's arithmetic, so both the CPU oracle's tests and the GPU path can take
their inputs from here without sharing any computation.

Shapes follow the layer described on "Mixture of Experts optimiza Transformers
y LLMs" (Keryc), section "¿Por qué MoEs importan ...": gpt-oss-20b with 4 of 32
experts active; "MoE (Mixture of Experts - Mezcla de Expertos)" (gotburnout
glossary), section 2 taxonomy: coarse 8-expert top-2 (Mixtral 8x7B) and fine
256-expert top-8 with one shared expert (DeepSeek V3).  The values are random:
no trained weights exist here and none are needed.

Draw rule (see synth.c): every tensor has a fixed tag; element i of a tensor is
``bf16(fp32(N_i * std))`` where ``N_i`` is a counter-based standard normal.
Weights therefore do not depend on T, and ``x`` for T tokens is the first T
rows of ``x`` for any larger T.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_lock = threading.Lock()

# tensor tags of the draw rule
TAG_W_G = 1
TAG_W_GATE_UP = 2
TAG_W_DOWN = 3
TAG_WS_GATE_UP = 4
TAG_WS_DOWN = 5
TAG_X = 6
TAG_ROUTER_BIAS = 7

WEIGHT_STD = 0.02
X_STD = 1.0


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so with gcc (OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.synth_key.restype = ctypes.c_uint64
            lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
            for name in ("synth_normal_bf16", "synth_normal_f32"):
                fn = getattr(lib, name)
                fn.restype = None
                fn.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                               ctypes.c_void_p]
            lib.synth_grid_bf16.restype = None
            lib.synth_grid_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                            ctypes.c_void_p]
            _lib = lib
    return _lib


def normal_bf16(shape, seed: int, tag: int, std: float, start: int = 0) -> torch.Tensor:
    """bf16 CPU tensor of ``shape`` drawn from stream (seed, tag), elements start.."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(tuple(shape), dtype=torch.bfloat16)
    if n:
        lib.synth_normal_bf16(lib.synth_key(seed, tag), start, n, float(std), out.data_ptr())
    return out


def normal_f32(shape, seed: int, tag: int, std: float, start: int = 0) -> torch.Tensor:
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(tuple(shape), dtype=torch.float32)
    if n:
        lib.synth_normal_f32(lib.synth_key(seed, tag), start, n, float(std), out.data_ptr())
    return out


def grid_bf16(shape, seed: int, tag: int) -> torch.Tensor:
    """bf16 tensor whose entries are multiples of 1/8 in [-2, 2]."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(tuple(shape), dtype=torch.bfloat16)
    if n:
        lib.synth_grid_bf16(lib.synth_key(seed, tag), 0, n, out.data_ptr())
    return out


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one MoE layer call.

    T tokens, D model width, E routed experts, k experts per token, F expert
    hidden width (d_ff), Fs shared-expert hidden width (0 = no shared expert).
    """
    T: int
    D: int
    E: int
    k: int
    F: int
    Fs: int = 0
    router_bias: bool = False
    # the router bias only moves the top-k selection, not the weights
    # (auxiliary-loss-free load balancing); needs router_bias
    bias_select: bool = False
    # expert weights (routed and shared) stored as E4M3 bytes with one fp32
    # scale per row, instead of bf16
    fp8: bool = False

    def with_T(self, T: int) -> "Shape":
        return dataclasses.replace(self, T=T)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    description: str
    T_list: tuple = ()


def skew_bias(E: int) -> torch.Tensor:
    """Per-expert router bias b_e = 3*ln(1/(e+1)^1.2) = -3.6*ln(e+1) (fp32).

    This is an *input* of the skewed-routing stress workload: it makes the
    expert loads Zipf-like so that one expert gets well over 40% of the
    assignments.
    """
    return torch.tensor([-3.6 * math.log(e + 1.0) for e in range(E)], dtype=torch.float32)


BALANCE_BIAS_STD = 0.5


def balance_bias(E: int, seed: int = 0) -> torch.Tensor:
    """Per-expert selection bias of the load-balancing mode: N(0, 0.5^2) fp32,
    drawn from stream (seed, TAG_ROUTER_BIAS).  Its spread is a fraction of
    the logits' (about 1 to 1.7 for the shapes here), so it moves a share of
    the selections without dominating them."""
    return normal_f32((E,), seed, TAG_ROUTER_BIAS, BALANCE_BIAS_STD)


def router_bias_for(shape: Shape, seed: int = 0) -> torch.Tensor | None:
    """The bias input a shape asks for: none, the skew bias (part of the
    logits) or the balancing bias (selection only)."""
    if not shape.router_bias:
        return None
    return balance_bias(shape.E, seed) if shape.bias_select else skew_bias(shape.E)


WORKLOADS = {
    "tiny": Workload("tiny", Shape(T=64, D=128, E=8, k=2, F=256),
                     "Tiny MoE layer: T=64, D=128, E=8, top-2, d_ff=256"),
    "mixtral_prefill": Workload("mixtral_prefill", Shape(T=4096, D=4096, E=8, k=2, F=14336),
                                "Mixtral-8x7B-shaped prefill: T=4096, D=4096, E=8, top-2, d_ff=14336"),
    "gptoss_decode": Workload("gptoss_decode", Shape(T=64, D=2880, E=32, k=4, F=2880),
                              "gpt-oss-20b-shaped decode: T in {1,8,32,64}, D=2880, E=32, top-4, d_ff=2880",
                              T_list=(1, 8, 32, 64)),
    "deepseek_fine": Workload("deepseek_fine", Shape(T=8192, D=7168, E=256, k=8, F=2048, Fs=2048),
                              "DeepSeek-V3-shaped fine-grained: T=8192, D=7168, 256 experts top-8 + 1 shared, d_ff=2048"),
    "mixtral_skewed": Workload("mixtral_skewed",
                               Shape(T=16384, D=4096, E=8, k=2, F=14336, router_bias=True),
                               "Skewed routing on the Mixtral shape at T=16384, bias -3.6*ln(e+1)"),
}


@dataclasses.dataclass
class LayerInputs:
    """All inputs of one layer call, as contiguous CPU (or device) tensors."""
    shape: Shape
    x: torch.Tensor                 # bf16 [T, D]
    w_g: torch.Tensor               # bf16 [E, D]
    w_gate_up: torch.Tensor         # bf16 [E, 2F, D]; rows 0..F-1 take the SiLU
    w_down: torch.Tensor            # bf16 [E, D, F]
    router_bias: torch.Tensor | None = None   # fp32 [E]
    ws_gate_up: torch.Tensor | None = None    # bf16 [2Fs, D]
    ws_down: torch.Tensor | None = None       # bf16 [D, Fs]
    # shape.fp8: the four expert tensors above are uint8 E4M3 codes, and these
    # hold the fp32 scale of each of their rows
    w_gate_up_scale: torch.Tensor | None = None   # [E, 2F]
    w_down_scale: torch.Tensor | None = None      # [E, D]
    ws_gate_up_scale: torch.Tensor | None = None  # [2Fs]
    ws_down_scale: torch.Tensor | None = None     # [D]

    def to(self, device) -> "LayerInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return LayerInputs(self.shape, mv(self.x), mv(self.w_g), mv(self.w_gate_up), mv(self.w_down),
                           mv(self.router_bias), mv(self.ws_gate_up), mv(self.ws_down),
                           mv(self.w_gate_up_scale), mv(self.w_down_scale), mv(self.ws_gate_up_scale),
                           mv(self.ws_down_scale))

    def with_x(self, x) -> "LayerInputs":
        return dataclasses.replace(self, x=x)


E4M3_MAX = 448.0


def quantize_rows_e4m3(w: torch.Tensor):
    """Per-row quantisation of a weight tensor [..., rows, cols] to E4M3 codes:
    scale = max|row| / 448 (1 for an all-zero row), code = E4M3 nearest to
    fp32(w / scale) (torch's float8_e4m3fn conversion, ties to even).  This only
    prepares inputs; the layer takes codes and scales as given."""
    wf = w.to(torch.float32)
    amax = wf.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (wf / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), scale.squeeze(-1).contiguous()


def make_weights(shape: Shape, seed: int = 0, std: float = WEIGHT_STD) -> LayerInputs:
    """Weights of the layer (x left empty); independent of T.  With shape.fp8
    the expert weights are the same draws quantised per row to E4M3."""
    E, D, F, Fs = shape.E, shape.D, shape.F, shape.Fs
    w_g = normal_bf16((E, D), seed, TAG_W_G, std)
    w_gu = normal_bf16((E, 2 * F, D), seed, TAG_W_GATE_UP, std)
    w_d = normal_bf16((E, D, F), seed, TAG_W_DOWN, std)
    ws_gu = ws_d = None
    if Fs:
        ws_gu = normal_bf16((2 * Fs, D), seed, TAG_WS_GATE_UP, std)
        ws_d = normal_bf16((D, Fs), seed, TAG_WS_DOWN, std)
    bias = router_bias_for(shape, seed)
    out = LayerInputs(shape, torch.empty((0, D), dtype=torch.bfloat16), w_g, w_gu, w_d, bias, ws_gu, ws_d)
    return quantize_inputs(out) if shape.fp8 else out


def quantize_inputs(inp: LayerInputs) -> LayerInputs:
    """The same layer with its expert weights quantised per row to E4M3."""
    out = dataclasses.replace(inp, shape=dataclasses.replace(inp.shape, fp8=True))
    out.w_gate_up, out.w_gate_up_scale = quantize_rows_e4m3(inp.w_gate_up)
    out.w_down, out.w_down_scale = quantize_rows_e4m3(inp.w_down)
    if inp.ws_gate_up is not None:
        out.ws_gate_up, out.ws_gate_up_scale = quantize_rows_e4m3(inp.ws_gate_up)
        out.ws_down, out.ws_down_scale = quantize_rows_e4m3(inp.ws_down)
    return out


def make_x(T: int, D: int, seed: int = 0, std: float = X_STD) -> torch.Tensor:
    return normal_bf16((T, D), seed, TAG_X, std)


def make_inputs(shape: Shape, seed: int = 0, weights: LayerInputs | None = None) -> LayerInputs:
    """Full inputs; pass ``weights`` to reuse one weight set across several T."""
    w = weights if weights is not None else make_weights(shape, seed)
    x = make_x(shape.T, shape.D, seed)
    return dataclasses.replace(w, shape=shape, x=x)


def make_grid_inputs(shape: Shape, seed: int = 0) -> LayerInputs:
    """Inputs whose entries are multiples of 1/8 in [-2, 2]: every router
    logit is then an exact small rational, so ties are exact and reproducible."""
    E, D, F, Fs = shape.E, shape.D, shape.F, shape.Fs
    ws_gu = ws_d = None
    if Fs:
        ws_gu = grid_bf16((2 * Fs, D), seed, TAG_WS_GATE_UP)
        ws_d = grid_bf16((D, Fs), seed, TAG_WS_DOWN)
    return LayerInputs(shape, grid_bf16((shape.T, D), seed, TAG_X), grid_bf16((E, D), seed, TAG_W_G),
                       grid_bf16((E, 2 * F, D), seed, TAG_W_GATE_UP), grid_bf16((E, D, F), seed, TAG_W_DOWN),
                       router_bias_for(shape, seed), ws_gu, ws_d)


# ---------------------------------------------------------------- size counts
def expert_params(shape: Shape) -> int:
    """Parameters of one routed expert: gate, up and down projections."""
    return 3 * shape.D * shape.F


def active_params(shape: Shape) -> int:
    """Parameters touched per token: k routed experts + router + shared expert."""
    return shape.k * expert_params(shape) + shape.D * shape.E + 3 * shape.D * shape.Fs


def total_params(shape: Shape) -> int:
    return shape.E * expert_params(shape) + shape.D * shape.E + 3 * shape.D * shape.Fs


def algorithmic_flops(shape: Shape) -> int:
    """2TDE (router) + 6TkDF (routed experts) + 6TDFs (shared expert)."""
    T, D, E, k, F, Fs = shape.T, shape.D, shape.E, shape.k, shape.F, shape.Fs
    return 2 * T * D * E + 6 * T * k * D * F + 6 * T * D * Fs


def algorithmic_bytes(shape: Shape, touched_experts: int) -> int:
    """Weights of experts actually used + router weights + x (bf16) + y (fp32)."""
    T, D, E, F, Fs = shape.T, shape.D, shape.E, shape.F, shape.Fs
    return (touched_experts * expert_params(shape) * 2 + 3 * D * Fs * 2 + E * D * 2
            + T * D * 2 + T * D * 4)


def gate_up_flops(shape: Shape) -> int:
    return 4 * shape.T * shape.k * shape.D * shape.F + 4 * shape.T * shape.D * shape.Fs


def down_flops(shape: Shape) -> int:
    return 2 * shape.T * shape.k * shape.D * shape.F + 2 * shape.T * shape.D * shape.Fs
