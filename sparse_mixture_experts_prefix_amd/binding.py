"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels.  torch supplies
device memory and the current stream; nothing here computes any part of the
layer, and there is no fallback: if libmoe.so is missing, or a tensor is not
on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_ALIGNMENT = -4
MOE_ERR_HIP = -5
MOE_ERR_SCRATCH = -6
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES: moe_forward_noalloc's array per GPU

EXPORTS = ("moe_workspace_size", "moe_block_m", "moe_forward", "moe_route", "moe_align",
           "moe_forward_routed", "moe_forward_timed", "moe_expert_load",
           "moe_backward_workspace_size", "moe_backward", "moe_train_workspace_size",
           "moe_forward_train", "moe_backward_saved", "moe_forward_noalloc", "moe_strerror")


class MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("libmoe error %d: %s" % (code, msg))
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("F", ctypes.c_int32), ("k", ctypes.c_int32), ("F_shared", ctypes.c_int32),
                ("has_router_bias", ctypes.c_int32), ("expert_begin", ctypes.c_int32),
                ("num_local_experts", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w_g", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("ws_gate_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
                ("w_gate_up_scale", ctypes.c_void_p), ("w_down_scale", ctypes.c_void_p),
                ("ws_gate_up_scale", ctypes.c_void_p), ("ws_down_scale", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dw_g", ctypes.c_void_p), ("d_bias", ctypes.c_void_p),
                ("dw_gate_up", ctypes.c_void_p), ("dw_down", ctypes.c_void_p),
                ("dws_gate_up", ctypes.c_void_p), ("dws_down", ctypes.c_void_p)]


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libmoe.so once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("libmoe.so is not built (%s); run __graft_entry__.build()" % path)
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            i32 = ctypes.c_int32
            lib.moe_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]
            lib.moe_block_m.argtypes = [ctypes.POINTER(Shape)]
            lib.moe_forward.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P, P, P,
                                        ctypes.c_size_t, P]
            lib.moe_route.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P, P]
            lib.moe_align.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
            lib.moe_forward_routed.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P,
                                               P, P, ctypes.c_size_t, P]
            lib.moe_forward_timed.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P,
                                              P, P, ctypes.c_size_t, P, P]
            lib.moe_expert_load.argtypes = [ctypes.POINTER(Shape), P, ctypes.c_size_t, P, P]
            lib.moe_backward_workspace_size.argtypes = [ctypes.POINTER(Shape),
                                                        ctypes.POINTER(ctypes.c_size_t)]
            lib.moe_backward.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P, P,
                                         ctypes.POINTER(Grads), P, ctypes.c_size_t, P]
            lib.moe_train_workspace_size.argtypes = [ctypes.POINTER(Shape),
                                                     ctypes.POINTER(ctypes.c_size_t)]
            lib.moe_forward_train.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P,
                                              P, P, ctypes.c_size_t, P]
            lib.moe_backward_saved.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P,
                                               P, ctypes.POINTER(Grads), P, ctypes.c_size_t, P,
                                               ctypes.c_size_t, P]
            lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Weights), P, P,
                                                P, P]
            lib.moe_strerror.argtypes = [ctypes.c_int]
            lib.moe_strerror.restype = ctypes.c_char_p
            for name in EXPORTS[:-1]:
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().moe_strerror(int(code)).decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise MoEError(rc, strerror(rc))
    return rc


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t, name, dtype, shape=None):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# moe_shape.weight_format values
WEIGHTS_BF16 = 0
WEIGHTS_FP8_E4M3 = 1   # uint8 E4M3 codes with one fp32 scale per row

# moe_shape.has_router_bias values
ROUTER_BIAS_NONE = 0
ROUTER_BIAS_LOGITS = 1   # the bias is part of the logits
ROUTER_BIAS_SELECT = 2   # the bias moves the top-k selection only


def bias_mode(router_bias, bias_select: bool) -> int:
    """has_router_bias for a call given its bias tensor (or None)."""
    if router_bias is None:
        if bias_select:
            raise ValueError("bias_select needs a router_bias")
        return ROUTER_BIAS_NONE
    return ROUTER_BIAS_SELECT if bias_select else ROUTER_BIAS_LOGITS


def make_shape(T, D, E, F, k, F_shared=0, has_router_bias=0, expert_begin=0,
               num_local_experts=0, weight_format=WEIGHTS_BF16) -> Shape:
    """moe_shape; has_router_bias is a ROUTER_BIAS_* value (a bool means
    none / logits); num_local_experts > 0 makes the call one expert-parallel
    shard holding experts expert_begin .. expert_begin+num_local_experts-1."""
    mode = (1 if has_router_bias else 0) if isinstance(has_router_bias, bool) else int(has_router_bias)
    return Shape(int(T), int(D), int(E), int(F), int(k), int(F_shared), mode,
                 int(expert_begin), int(num_local_experts), int(weight_format))


def workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def block_m(shape: Shape) -> int:
    return _check(load_library().moe_block_m(ctypes.byref(shape)))


def _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, has_bias, n_experts=None, expert_begin=None):
    """Shape of a layer call; the call is a shard when the expert weights hold
    fewer experts than the router scores (n_experts) or expert_begin is given.
    uint8 expert weights are E4M3 codes."""
    T, D = x.shape
    E_loc, twoF, D2 = w_gate_up.shape
    F = twoF // 2
    Fs = 0 if ws_gate_up is None else ws_gate_up.shape[0] // 2
    E = E_loc if n_experts is None else int(n_experts)
    fmt = WEIGHTS_FP8_E4M3 if w_gate_up.dtype == torch.uint8 else WEIGHTS_BF16
    if expert_begin is None and E == E_loc:
        return make_shape(T, D, E, F, k, Fs, has_bias, weight_format=fmt)
    return make_shape(T, D, E, F, k, Fs, has_bias, expert_begin or 0, E_loc, fmt)


def alloc_workspace(shape: Shape, device) -> torch.Tensor:
    return torch.empty(max(workspace_size(shape), 1), dtype=torch.uint8, device=device)


def _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down, scales=None) -> Weights:
    sc = tuple(scales) if scales is not None else (None, None, None, None)
    return Weights(_ptr(x), _ptr(w_g), _ptr(router_bias), _ptr(w_gate_up), _ptr(w_down),
                   _ptr(ws_gate_up), _ptr(ws_down), *[_ptr(t) for t in sc])


def _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down, scales=None):
    """Checks the layer tensors.  Expert weights are all bf16, or all uint8
    E4M3 codes with scales = (w_gate_up_scale [E,2F], w_down_scale [E,D],
    ws_gate_up_scale [2Fs] or None, ws_down_scale [D] or None), fp32."""
    _dev(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [T, D]")
    T, D = x.shape
    wdt = w_gate_up.dtype if w_gate_up is not None else torch.bfloat16
    if wdt not in (torch.bfloat16, torch.uint8):
        raise ValueError("expert weights must be bf16 or uint8 (E4M3 codes)")
    _dev(w_gate_up, "w_gate_up", wdt)
    if w_gate_up.dim() != 3 or w_gate_up.shape[2] != D or w_gate_up.shape[1] % 2:
        raise ValueError("w_gate_up must be [E, 2F, D]")
    E, twoF, _ = w_gate_up.shape
    _dev(w_down, "w_down", wdt, (E, D, twoF // 2))
    if (ws_gate_up is None) != (ws_down is None):
        raise ValueError("ws_gate_up and ws_down go together")
    if ws_gate_up is not None:
        _dev(ws_gate_up, "ws_gate_up", wdt)
        if ws_gate_up.dim() != 2 or ws_gate_up.shape[1] != D or ws_gate_up.shape[0] % 2:
            raise ValueError("ws_gate_up must be [2Fs, D]")
        _dev(ws_down, "ws_down", wdt, (D, ws_gate_up.shape[0] // 2))
    tensors = [w_gate_up, w_down, ws_gate_up, ws_down]
    if wdt == torch.uint8:
        if scales is None or len(scales) != 4:
            raise ValueError("E4M3 weights need scales=(w_gate_up_scale, w_down_scale, "
                             "ws_gate_up_scale, ws_down_scale)")
        sgu, sdn, ssgu, ssdn = scales
        _dev(sgu, "w_gate_up_scale", torch.float32, (E, twoF))
        _dev(sdn, "w_down_scale", torch.float32, (E, D))
        if ws_gate_up is not None:
            _dev(ssgu, "ws_gate_up_scale", torch.float32, (ws_gate_up.shape[0],))
            _dev(ssdn, "ws_down_scale", torch.float32, (D,))
        tensors += [sgu, sdn, ssgu, ssdn]
    elif scales is not None and any(t is not None for t in scales):
        raise ValueError("scales are only for uint8 (E4M3) weights")
    for t in tensors:
        if t is not None and t.device != x.device:
            raise ValueError("all tensors must be on one device")
    return T, D, E, twoF // 2


def moe_forward(x, w_g, w_gate_up, w_down, k, router_bias=None, ws_gate_up=None, ws_down=None, *,
                y=None, topk_ids=None, topk_w=None, workspace=None, expert_begin=None,
                bias_select=False, scales=None):
    """Whole MoE layer.  Returns y (fp32 [T, D]).

    bias_select: router_bias moves only the top-k selection (load balancing);
    the weights are the softmax of the plain chosen logits.

    uint8 expert weights are E4M3 codes; then scales = (w_gate_up_scale
    [E,2F], w_down_scale [E,D], ws_gate_up_scale [2Fs], ws_down_scale [D])
    gives the fp32 scale of every weight row.

    Optional preallocated outputs (y, topk_ids int32 [T,k], topk_w fp32 [T,k])
    and workspace (uint8, >= workspace_size bytes) avoid any allocation here.
    Expert-parallel shard: pass w_gate_up / w_down of experts expert_begin ..
    expert_begin + n - 1 only (w_g still covers all E); y is then the shard's
    part of the layer.
    """
    T, D, E_loc, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    _dev(w_g, "w_g", torch.bfloat16)
    E = w_g.shape[0]
    _dev(w_g, "w_g", torch.bfloat16, (E, D))
    if E_loc != E and expert_begin is None:
        raise ValueError("w_gate_up holds %d of %d experts: pass expert_begin" % (E_loc, E))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, bias_mode(router_bias, bias_select), E,
                         expert_begin)
    if y is None:
        y = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32, (T, D))
    if topk_ids is not None:
        _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, (T, k))
    if workspace is None:
        workspace = alloc_workspace(shape, x.device)
    _dev(workspace, "workspace", torch.uint8)
    w = _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    _check(load_library().moe_forward(ctypes.byref(shape), ctypes.byref(w), _ptr(y), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(workspace), workspace.numel(),
                                      _stream(x.device)))
    return y


def moe_forward_noalloc(x, w_g, w_gate_up, w_down, k, router_bias=None, ws_gate_up=None,
                        ws_down=None, *, y, topk_ids=None, topk_w=None, expert_begin=None,
                        bias_select=False, scales=None):
    """moe_forward whose workspace is the library's static per-GPU array
    (moe_forward_noalloc in moe.h): nothing is allocated, here or in the
    library, so the outputs are preallocated (y fp32 [T, D]; topk_ids int32
    [T, k] and topk_w fp32 [T, k], or None).  Calls that overlap on one GPU
    race on that array.  Raises MoEError(MOE_ERR_SCRATCH) for shapes whose
    workspace exceeds it.  Returns y."""
    T, D, E_loc, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    _dev(w_g, "w_g", torch.bfloat16)
    E = w_g.shape[0]
    _dev(w_g, "w_g", torch.bfloat16, (E, D))
    if E_loc != E and expert_begin is None:
        raise ValueError("w_gate_up holds %d of %d experts: pass expert_begin" % (E_loc, E))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, bias_mode(router_bias, bias_select), E,
                         expert_begin)
    _dev(y, "y", torch.float32, (T, D))
    if topk_ids is not None:
        _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, (T, k))
    w = _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    _check(load_library().moe_forward_noalloc(ctypes.byref(shape), ctypes.byref(w), _ptr(y),
                                              _ptr(topk_ids), _ptr(topk_w), _stream(x.device)))
    return y


def moe_route(x, w_g, k, router_bias=None, *, topk_ids=None, topk_w=None, bias_select=False):
    """Router only.  Returns (topk_ids int32 [T,k], topk_w fp32 [T,k])."""
    _dev(x, "x", torch.bfloat16)
    T, D = x.shape
    _dev(w_g, "w_g", torch.bfloat16)
    E = w_g.shape[0]
    _dev(w_g, "w_g", torch.bfloat16, (E, D))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    shape = make_shape(T, D, E, 8, k, 0, bias_mode(router_bias, bias_select))
    w = _weights(x, w_g, router_bias, None, None, None, None)
    _check(load_library().moe_route(ctypes.byref(shape), ctypes.byref(w), _ptr(topk_ids),
                                    _ptr(topk_w), _stream(x.device)))
    return topk_ids, topk_w


def moe_align(topk_ids, E: int, block_m_: int, shared_rows: int = 0):
    """Expert grouping of a routing (int32 [T, k] on the GPU).  Returns a dict of
    int32 GPU tensors sized to their upper bounds plus ``n_tiles`` (1 element)."""
    _dev(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    G = E + (1 if shared_rows > 0 else 0)
    cap = T * k + G * (block_m_ - 1) + shared_rows
    dev = topk_ids.device

    def z(n, fill=0):
        return torch.full((max(n, 1),), fill, dtype=torch.int32, device=dev)

    out = dict(counts=z(G), offsets=z(G + 1), padded=z(G + 1), sorted_assign=z(T * k),
               row_of=z(T * k), row_token=z(cap, -7), tile_group=z(cap // block_m_ + 1, -7),
               n_tiles=z(1))
    _check(load_library().moe_align(
        _ptr(topk_ids), T, k, E, block_m_, shared_rows, _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["padded"]), _ptr(out["sorted_assign"]), _ptr(out["row_of"]), _ptr(out["row_token"]),
        _ptr(out["tile_group"]), _ptr(out["n_tiles"]), _stream(dev)))
    return out


def moe_forward_routed(x, w_gate_up, w_down, topk_ids, topk_w, ws_gate_up=None, ws_down=None, *,
                       y=None, workspace=None, n_experts=None, expert_begin=None, scales=None):
    """The layer under a given routing (topk_ids int32 [T,k], topk_w fp32 [T,k]).
    For a shard, n_experts is the router's expert count and expert_begin the
    first held expert.  scales: as in moe_forward."""
    T, D, E, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    k = topk_ids.shape[1]
    _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, False, n_experts, expert_begin)
    if y is None:
        y = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32, (T, D))
    if workspace is None:
        workspace = alloc_workspace(shape, x.device)
    w = _weights(x, None, None, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    _check(load_library().moe_forward_routed(ctypes.byref(shape), ctypes.byref(w), _ptr(topk_ids),
                                             _ptr(topk_w), _ptr(y), _ptr(workspace),
                                             workspace.numel(), _stream(x.device)))
    return y


def layer_shape(x, w_g, w_gate_up, k, ws_gate_up=None, router_bias=None, *, bias_select=False,
                expert_begin=None) -> Shape:
    """The moe_shape moe_forward builds for these tensors (for workspace_size
    and moe_expert_load)."""
    return _layer_shape(x, w_gate_up, None, k, ws_gate_up, bias_mode(router_bias, bias_select),
                        w_g.shape[0], expert_begin)


def moe_expert_load(shape: Shape, workspace, counts=None):
    """Per-expert assignment counts of the last layer call on ``workspace``
    with ``shape``: int32 [G] on the workspace's device, G = held experts (+1
    for the shared expert, whose entry is T)."""
    G = (shape.num_local_experts or shape.E) + (1 if shape.F_shared > 0 else 0)
    _dev(workspace, "workspace", torch.uint8)
    if counts is None:
        counts = torch.empty(G, dtype=torch.int32, device=workspace.device)
    _dev(counts, "counts", torch.int32, (G,))
    _check(load_library().moe_expert_load(ctypes.byref(shape), _ptr(workspace), workspace.numel(),
                                          _ptr(counts), _stream(workspace.device)))
    return counts


def backward_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_backward_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def train_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_train_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def moe_forward_train(x, w_g, w_gate_up, w_down, k, router_bias=None, ws_gate_up=None,
                      ws_down=None, *, bias_select=False, y=None, topk_ids=None, topk_w=None,
                      workspace=None):
    """moe_forward that keeps the rows' grouping and g | u in its workspace for
    moe_backward(..., saved=workspace).  Returns (y, topk_ids, topk_w, workspace)."""
    T, D, E, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down)
    _dev(w_g, "w_g", torch.bfloat16, (E, D))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, bias_mode(router_bias, bias_select))
    dev = x.device
    y = torch.empty((T, D), dtype=torch.float32, device=dev) if y is None else y
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _dev(y, "y", torch.float32, (T, D))
    _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if workspace is None:
        workspace = torch.empty(max(train_workspace_size(shape), 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    w = _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down)
    _check(load_library().moe_forward_train(ctypes.byref(shape), ctypes.byref(w), _ptr(y),
                                            _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                                            workspace.numel(), _stream(dev)))
    return y, topk_ids, topk_w, workspace


def moe_backward(x, w_g, w_gate_up, w_down, k, topk_ids, topk_w, dy, router_bias=None,
                 ws_gate_up=None, ws_down=None, *, bias_select=False, workspace=None, grads=None,
                 saved=None):
    """Gradients of sum <dy, y> for the routing (topk_ids, topk_w) of a forward
    call with the same tensors.  Returns a dict of fp32 tensors dx, dw_g,
    d_bias, dw_gate_up, dw_down (and dws_gate_up, dws_down with a shared
    expert); ``grads`` may hold preallocated ones.  ``saved``: the workspace of
    the moe_forward_train call that returned this routing (moe_backward_saved)."""
    T, D, E, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down)
    _dev(w_g, "w_g", torch.bfloat16, (E, D))
    _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    _dev(dy, "dy", torch.float32, (T, D))
    if router_bias is not None:
        _dev(router_bias, "router_bias", torch.float32, (E,))
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, bias_mode(router_bias, bias_select))
    Fs = shape.F_shared
    dev = x.device
    sizes = dict(dx=(T, D), dw_g=(E, D), d_bias=(E,), dw_gate_up=(E, 2 * F, D), dw_down=(E, D, F))
    if Fs:
        sizes.update(dws_gate_up=(2 * Fs, D), dws_down=(D, Fs))
    out = dict(grads or {})
    for name, shp in sizes.items():
        if name not in out:
            out[name] = torch.empty(shp, dtype=torch.float32, device=dev)
        _dev(out[name], name, torch.float32, shp)
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_size(shape), 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    gr = Grads(*[_ptr(out.get(n)) for n, _ in Grads._fields_])
    w = _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down)
    lib = load_library()
    if saved is None:
        _check(lib.moe_backward(ctypes.byref(shape), ctypes.byref(w), _ptr(topk_ids), _ptr(topk_w),
                                _ptr(dy), ctypes.byref(gr), _ptr(workspace), workspace.numel(),
                                _stream(dev)))
    else:
        _dev(saved, "saved", torch.uint8)
        _check(lib.moe_backward_saved(ctypes.byref(shape), ctypes.byref(w), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(dy), ctypes.byref(gr), _ptr(saved),
                                      saved.numel(), _ptr(workspace), workspace.numel(),
                                      _stream(dev)))
    return out


# the C names, one to one
moe_workspace_size = workspace_size
moe_backward_workspace_size = backward_workspace_size
moe_train_workspace_size = train_workspace_size
moe_block_m = block_m
moe_strerror = strerror


# ------------------------------------------------------------------ timing
class HipEvents:
    """A few raw hipEvent_t handles from the HIP runtime already loaded in this
    process (the one torch uses), for moe_forward_timed."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self._hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            self.handles.append(h.value)
        self.array = (ctypes.c_void_p * n)(*self.handles)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float(0.0)
        self._hip.hipEventSynchronize(ctypes.c_void_p(self.handles[j]))
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[i]),
                                           ctypes.c_void_p(self.handles[j]))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(ctypes.c_void_p(h))
        self.handles = []


def moe_forward_timed(events: HipEvents, x, w_g, w_gate_up, w_down, k, router_bias=None,
                      ws_gate_up=None, ws_down=None, *, y, topk_ids, topk_w, workspace,
                      expert_begin=None, bias_select=False, scales=None):
    """moe_forward recording events[0..5] around its five kernels (all buffers preallocated)."""
    T, D, E, F = _check_layer(x, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    shape = _layer_shape(x, w_gate_up, w_down, k, ws_gate_up, bias_mode(router_bias, bias_select),
                         w_g.shape[0], expert_begin)
    w = _weights(x, w_g, router_bias, w_gate_up, w_down, ws_gate_up, ws_down, scales)
    lib = load_library()
    _check(lib.moe_forward_timed(ctypes.byref(shape), ctypes.byref(w), _ptr(y), _ptr(topk_ids),
                                 _ptr(topk_w), _ptr(workspace), workspace.numel(), _stream(x.device),
                                 ctypes.cast(events.array, ctypes.c_void_p)))
    return y
