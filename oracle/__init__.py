"""CPU oracle of one sparse-MoE SwiGLU layer forward pass (ctypes over oracle.c).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
and its Python binding never import it and share no code with it.

Parity pins of each function (what ties it to something other than itself)
are in ``tests/test_oracle_*.py``:
  route   -- exact rational logits on grid inputs, numpy stable argsort,
             softmax-over-all-then-renormalise, sum-to-one, k=1, shift invariance
  experts -- float64 dense evaluation of every expert on every token, a
             textbook dense SwiGLU FFN at E=1, identical experts, k=E soft
             mixture, relabelling, token independence, exact power-of-two scaling,
             hand-computed closed-form fixtures under tests/golden/
  align   -- Python ``sorted`` of (expert, assignment) pairs and the padding
             invariants
Absolute layer outputs at the named workloads have no printed values on the
pages; beyond the pins above they are "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 -fopenmp (no BLAS, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
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
            lib.oracle_route.restype = ctypes.c_int
            lib.oracle_route.argtypes = [_p, _p, _p, _i64, _i32, _i32, _i32, _p, _p, _p, _p]
            lib.oracle_route_mode.restype = ctypes.c_int
            lib.oracle_route_mode.argtypes = [_p, _p, _p, _i32, _i64, _i32, _i32, _i32, _p, _p, _p,
                                              _p]
            lib.oracle_experts.restype = ctypes.c_int
            lib.oracle_experts.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p,
                                           _p, _i64, _p, _p]
            lib.oracle_experts_shard.restype = ctypes.c_int
            lib.oracle_experts_shard.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _p, _p, _p, _i64, _p, _p]
            lib.oracle_experts_q.restype = ctypes.c_int
            lib.oracle_experts_q.argtypes = [_p, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _i32, _i32,
                                             _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i64, _p, _p]
            lib.oracle_backward.restype = ctypes.c_int
            lib.oracle_backward.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
            lib.oracle_e4m3_decode.restype = None
            lib.oracle_e4m3_decode.argtypes = [_p, _i64, _p]
            lib.oracle_align.restype = ctypes.c_int
            lib.oracle_align.argtypes = [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                         _i64, _p, _p]
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _bf16_ptr(t):
    """Pointer to a contiguous CPU bf16 tensor (or None). Keeps no copy."""
    if t is None:
        return None, None
    if t.device.type != "cpu" or t.dtype != torch.bfloat16:
        raise TypeError("oracle takes CPU bfloat16 tensors")
    t = t.contiguous()
    return t.data_ptr(), t


def _w_ptr(t):
    """Pointer to a contiguous CPU weight tensor: bf16, or uint8 E4M3 codes."""
    if t is None:
        return None, None
    if t.device.type != "cpu" or t.dtype not in (torch.bfloat16, torch.uint8):
        raise TypeError("oracle takes CPU bfloat16 or uint8 (E4M3) weight tensors")
    t = t.contiguous()
    return t.data_ptr(), t


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array) as float64, from the format's definition."""
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode(c.ctypes.data, c.size, out.ctypes.data)
    return out


def _f32_ptr(t):
    if t is None:
        return None, None
    t = t.detach().to("cpu", torch.float32).contiguous()
    return t.data_ptr(), t


def bias_mode(router_bias, select_only: bool) -> int:
    """0 no bias, 1 bias inside the logits, 2 selection-only bias."""
    if router_bias is None:
        return 0
    return 2 if select_only else 1


def route(x, w_g, router_bias, k: int, select_only: bool = False):
    """Router for every row of x.  With select_only the bias moves only the
    top-k selection; the weights are the softmax of the plain chosen logits.

    Returns (ids int32 [T,k], p float64 [T,k], margin float64 [T] on the
    selection keys, logits float32 [T,E] without a selection-only bias).
    """
    lib = _load()
    T, D = x.shape
    E = w_g.shape[0]
    px, kx = _bf16_ptr(x)
    pw, kw = _bf16_ptr(w_g)
    pb, kb = _f32_ptr(router_bias)
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, k), np.int32)
    p = np.empty((T, k), np.float64)
    margin = np.empty((T,), np.float64)
    rc = lib.oracle_route_mode(px, pw, pb, bias_mode(router_bias, select_only), T, D, E, k,
                               logits.ctypes.data, ids.ctypes.data, p.ctypes.data,
                               margin.ctypes.data)
    if rc:
        raise ValueError("oracle_route_mode failed: %d" % rc)
    return ids, p, margin, logits


def experts(inp, ids, p, tokens=None, count_macs: bool = False, expert_begin: int = 0,
            n_local=None):
    """Expert outputs y [n, D] (float64) for ``tokens`` (default: all rows of x)
    under the routing (ids [T,k] int, p [T,k] float).

    With ``n_local`` set, ``inp.w_gate_up`` / ``inp.w_down`` hold only experts
    expert_begin .. expert_begin+n_local-1 of the ``inp.shape.E`` the router
    scores, and only slots routed to them contribute (one expert-parallel
    shard); the shared expert is included when ``inp`` carries it."""
    lib = _load()
    s = inp.shape
    px, kx = _bf16_ptr(inp.x)
    fp8 = inp.w_gate_up.dtype == torch.uint8
    pgu, k1 = _w_ptr(inp.w_gate_up)
    pdn, k2 = _w_ptr(inp.w_down)
    psgu, k3 = _w_ptr(inp.ws_gate_up)
    psdn, k4 = _w_ptr(inp.ws_down)
    q1, r1 = _f32_ptr(inp.w_gate_up_scale if fp8 else None)
    q2, r2 = _f32_ptr(inp.w_down_scale if fp8 else None)
    q3, r3 = _f32_ptr(inp.ws_gate_up_scale if fp8 else None)
    q4, r4 = _f32_ptr(inp.ws_down_scale if fp8 else None)
    ids = np.ascontiguousarray(ids, np.int32)
    p = np.ascontiguousarray(p, np.float64)
    T = inp.x.shape[0]
    if ids.shape != (T, s.k) or p.shape != (T, s.k):
        raise ValueError("routing shape mismatch")
    nl = s.E if n_local is None else int(n_local)
    if inp.w_gate_up.shape[0] != nl or inp.w_down.shape[0] != nl:
        raise ValueError("expert weights hold %d experts, expected %d" % (inp.w_gate_up.shape[0], nl))
    if tokens is None:
        tok = None
        n = T
    else:
        tok = np.ascontiguousarray(tokens, np.int64)
        if tok.size and (tok.min() < 0 or tok.max() >= T):
            raise ValueError("token index out of range")
        n = tok.size
    y = np.empty((n, s.D), np.float64)
    macs = ctypes.c_int64(0)
    rc = lib.oracle_experts_q(px, pgu, pdn, psgu, psdn, 1 if fp8 else 0, q1, q2, q3, q4, s.D, s.E,
                              int(expert_begin), nl, s.F, s.k, s.Fs, ids.ctypes.data,
                              p.ctypes.data, None if tok is None else tok.ctypes.data, n,
                              y.ctypes.data, ctypes.byref(macs))
    if rc:
        raise ValueError("oracle_experts_q failed: %d" % rc)
    return (y, macs.value) if count_macs else y


def forward(inp):
    """Whole layer for every token: route every row of x, then run its experts.
    Returns (y float64 [T,D], ids, p, margin)."""
    ids, p, margin, _ = route(inp.x, inp.w_g, inp.router_bias, inp.shape.k,
                              select_only=inp.shape.bias_select)
    return experts(inp, ids, p), ids, p, margin


def backward(inp, ids, p, dy):
    """Gradients of sum_t <dy[t], y[t]> for the routing (ids [T,k], p [T,k]):
    a dict of float64 arrays dx [T,D], dw_g [E,D], d_bias [E] (zero unless the
    bias is part of the logits), dw_gate_up [E,2F,D], dw_down [E,D,F],
    dws_gate_up [2Fs,D] / dws_down [D,Fs] (shared expert only) and dp [T,k]
    (<dy, expert output> per slot).  bf16 expert weights only."""
    lib = _load()
    s = inp.shape
    T = inp.x.shape[0]
    if inp.w_gate_up.dtype != torch.bfloat16:
        raise TypeError("the backward oracle takes bf16 expert weights")
    px, kx = _bf16_ptr(inp.x)
    pg, kg = _bf16_ptr(inp.w_g)
    pgu, k1 = _bf16_ptr(inp.w_gate_up)
    pdn, k2 = _bf16_ptr(inp.w_down)
    psgu, k3 = _bf16_ptr(inp.ws_gate_up)
    psdn, k4 = _bf16_ptr(inp.ws_down)
    ids = np.ascontiguousarray(ids, np.int32)
    p = np.ascontiguousarray(p, np.float64)
    dyf = np.ascontiguousarray(dy, np.float32)
    if ids.shape != (T, s.k) or p.shape != (T, s.k) or dyf.shape != (T, s.D):
        raise ValueError("shape mismatch")
    out = dict(dx=np.empty((T, s.D)), dw_g=np.empty((s.E, s.D)), d_bias=np.empty(s.E),
               dw_gate_up=np.empty((s.E, 2 * s.F, s.D)), dw_down=np.empty((s.E, s.D, s.F)),
               dp=np.empty((T, s.k)))
    if s.Fs:
        out["dws_gate_up"] = np.empty((2 * s.Fs, s.D))
        out["dws_down"] = np.empty((s.D, s.Fs))
    mode = 1 if (inp.router_bias is not None and not s.bias_select) else 0

    def ptr(name):
        return out[name].ctypes.data if name in out else None

    rc = lib.oracle_backward(px, pg, pgu, pdn, psgu, psdn, T, s.D, s.E, s.F, s.k, s.Fs, mode,
                             ids.ctypes.data, p.ctypes.data, dyf.ctypes.data, ptr("dx"),
                             ptr("dw_g"), ptr("d_bias"), ptr("dw_gate_up"), ptr("dw_down"),
                             ptr("dws_gate_up"), ptr("dws_down"), ptr("dp"))
    if rc:
        raise ValueError("oracle_backward failed: %d" % rc)
    return out


def align(ids, E: int, block_m: int, shared: bool = False):
    """Group assignments by expert (stable in assignment order) with BM-padded groups.

    Returns a dict of int32 arrays: counts, offsets, padded, sorted_assign,
    row_of, row_token (length padded[G]), tile_group (length n_tiles), n_tiles.
    """
    lib = _load()
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    G = E + (1 if shared else 0)
    cap = T * k + G * (block_m - 1) + (T if shared else 0)
    counts = np.zeros(G, np.int32)
    offsets = np.zeros(G + 1, np.int32)
    padded = np.zeros(G + 1, np.int32)
    sorted_assign = np.zeros(T * k, np.int32)
    row_of = np.zeros(T * k, np.int32)
    row_token = np.zeros(max(cap, 1), np.int32)
    tile_group = np.zeros(max(cap // block_m + 1, 1), np.int32)
    n_tiles = ctypes.c_int32(0)
    rc = lib.oracle_align(ids.ctypes.data, T, k, E, block_m, 1 if shared else 0,
                          counts.ctypes.data, offsets.ctypes.data, padded.ctypes.data,
                          sorted_assign.ctypes.data, row_of.ctypes.data, row_token.ctypes.data,
                          cap, tile_group.ctypes.data, ctypes.byref(n_tiles))
    if rc:
        raise ValueError("oracle_align failed: %d" % rc)
    nt = n_tiles.value
    return dict(counts=counts, offsets=offsets, padded=padded, sorted_assign=sorted_assign,
                row_of=row_of, row_token=row_token[:padded[G]].copy(),
                tile_group=tile_group[:nt].copy(), n_tiles=nt)
