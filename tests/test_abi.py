"""The C ABI without a GPU: the library loads, exports every symbol moe.h
declares, and its host-side checks return the documented codes before any
launch (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("sparse_mixture_experts_prefix_amd")
from sparse_mixture_experts_prefix_amd import binding as B  # noqa: E402
from sparse_mixture_experts_prefix_amd import build as native  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(native.LIB_PATH):
        native.build()
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_forward", "moe_route", "moe_align", "moe_forward_routed", "moe_workspace_size",
              "moe_block_m", "moe_strerror"):
        assert n in names


def test_every_export_has_its_argument_types():
    """Pointers and sizes are 64-bit: a missing argtypes would pass them as C int."""
    lib = B.load_library()
    for n in B.EXPORTS:
        assert getattr(lib, n).argtypes is not None, n


def test_router_bias_modes_match_the_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (MOE_ROUTER_BIAS_[A-Z]+) (\d+)", text))
    assert defs == {"MOE_ROUTER_BIAS_NONE": str(B.ROUTER_BIAS_NONE),
                    "MOE_ROUTER_BIAS_LOGITS": str(B.ROUTER_BIAS_LOGITS),
                    "MOE_ROUTER_BIAS_SELECT": str(B.ROUTER_BIAS_SELECT)}


def test_weight_formats_match_the_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (MOE_WEIGHTS_[A-Z0-9_]+) (\d+)", text))
    assert defs == {"MOE_WEIGHTS_BF16": str(B.WEIGHTS_BF16),
                    "MOE_WEIGHTS_FP8_E4M3": str(B.WEIGHTS_FP8_E4M3)}


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(B.EXPORTS)


def _shape(**kw):
    d = dict(T=64, D=128, E=8, F=256, k=2, F_shared=0, has_router_bias=0)
    d.update(kw)
    return B.Shape(**d)


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _weights(**kw):
    d = dict(x=FAKE, w_g=FAKE, router_bias=None, w_gate_up=FAKE, w_down=FAKE, ws_gate_up=None,
             ws_down=None)
    d.update(kw)
    return B.Weights(**d)


def _fwd(lib, shape, w, y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.moe_forward(ctypes.byref(shape), ctypes.byref(w), y, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), B.MOE_ERR_INVALID_ARG), (dict(k=9, E=16), B.MOE_ERR_UNSUPPORTED),
    (dict(k=3, E=2), B.MOE_ERR_INVALID_ARG), (dict(E=257), B.MOE_ERR_UNSUPPORTED),
    (dict(D=100), B.MOE_ERR_INVALID_ARG), (dict(F=12), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG), (dict(F_shared=4), B.MOE_ERR_INVALID_ARG),
    # expert-parallel shards: the held range must lie inside [0, E)
    (dict(expert_begin=6, num_local_experts=3), B.MOE_ERR_INVALID_ARG),
    (dict(expert_begin=-1, num_local_experts=2), B.MOE_ERR_INVALID_ARG),
    (dict(expert_begin=2, num_local_experts=0), B.MOE_ERR_INVALID_ARG),
    (dict(num_local_experts=-1), B.MOE_ERR_INVALID_ARG),
    # router bias modes are 0 (none), 1 (in the logits), 2 (selection only)
    (dict(has_router_bias=3), B.MOE_ERR_INVALID_ARG),
    (dict(has_router_bias=-1), B.MOE_ERR_INVALID_ARG),
    (dict(weight_format=2), B.MOE_ERR_INVALID_ARG),
    (dict(T=1 << 30, k=8), B.MOE_ERR_UNSUPPORTED)])
def test_shape_errors(lib, kw, code):
    assert _fwd(lib, _shape(**kw), _weights()) == code
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(_shape(**kw)), ctypes.byref(n)) == code


def test_pointer_errors(lib):
    s = _shape()
    assert _fwd(lib, s, _weights(x=None)) == B.MOE_ERR_INVALID_ARG
    assert _fwd(lib, s, _weights(w_down=None)) == B.MOE_ERR_INVALID_ARG
    assert _fwd(lib, s, _weights(), y=None) == B.MOE_ERR_INVALID_ARG
    assert _fwd(lib, s, _weights(x=FAKE + 8)) == B.MOE_ERR_ALIGNMENT
    assert _fwd(lib, s, _weights(), y=FAKE + 4) == B.MOE_ERR_ALIGNMENT
    assert _fwd(lib, _shape(has_router_bias=1), _weights()) == B.MOE_ERR_INVALID_ARG
    assert _fwd(lib, _shape(has_router_bias=2), _weights()) == B.MOE_ERR_INVALID_ARG
    assert _fwd(lib, _shape(F_shared=64), _weights()) == B.MOE_ERR_INVALID_ARG


def test_workspace_too_small(lib):
    s = _shape()
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    assert _fwd(lib, s, _weights(), ws_bytes=n.value - 1) == B.MOE_ERR_WORKSPACE


def test_zero_tokens_is_a_no_op(lib):
    # T = 0 returns before any launch, even with no x or y
    assert _fwd(lib, _shape(T=0), _weights(x=None), y=None, ws=None) == 0


def test_workspace_and_block_m(lib):
    s = _shape(T=4096, D=4096, E=8, F=14336, k=2)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    bm = lib.moe_block_m(ctypes.byref(s))
    assert bm in (16, 32, 64, 128, 256)
    rows = 4096 * 2 + 8 * (bm - 1)
    # at least H (bf16) and Yp (fp32) for every padded row
    assert n.value >= rows * (14336 * 2 + 4096 * 4)
    assert n.value < 2 * rows * (14336 * 2 + 4096 * 4)


def test_align_argument_errors(lib):
    P = FAKE
    assert lib.moe_align(P, 10, 2, 8, 0, 0, P, P, P, P, P, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_align(P, 10, 9, 16, 16, 0, P, P, P, P, P, P, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_align(P, 10, 2, 8, 16, 0, None, P, P, P, P, P, P, P, None) == B.MOE_ERR_INVALID_ARG


def test_weights_struct_matches_header():
    """moe_weights is pointers only, in the header's order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct moe_weights \{(.*?)\} moe_weights;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == [f[0] for f in B.Weights._fields_]
    assert ctypes.sizeof(B.Weights) == 8 * len(names)


def test_shape_struct_matches_header():
    """moe_shape is int32 fields in the header's order."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct moe_shape \{(.*?)\} moe_shape;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"int32_t\s+(\w+);", body)
    assert names == [f[0] for f in B.Shape._fields_]
    assert ctypes.sizeof(B.Shape) == 4 * len(names)


def test_shard_workspace_is_smaller(lib):
    full = B.workspace_size(_shape(T=4096, E=64, k=2))
    shard = B.workspace_size(_shape(T=4096, E=64, k=2, expert_begin=8, num_local_experts=8))
    assert 0 < shard < full
    assert B.workspace_size(_shape(T=4096, E=64, k=2, expert_begin=0, num_local_experts=64)) == full


def test_noalloc_rejects_shapes_beyond_its_array(lib):
    """moe_forward_noalloc refuses, before touching any device, a shape whose
    workspace exceeds the static array (the Mixtral-shaped prefill layer needs
    about 0.5 GB), and checks its arguments as moe_forward does."""
    big = _shape(T=4096, D=4096, E=8, F=14336, k=2)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0
    assert n.value > B.STATIC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), ctypes.byref(_weights()), FAKE, None, None,
                                   None) == B.MOE_ERR_SCRATCH
    small = _shape()
    assert lib.moe_forward_noalloc(ctypes.byref(small), ctypes.byref(_weights(x=None)), FAKE, None,
                                   None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_noalloc(ctypes.byref(small), ctypes.byref(_weights()), FAKE + 4, None,
                                   None, None) == B.MOE_ERR_ALIGNMENT
    assert lib.moe_forward_noalloc(ctypes.byref(_shape(T=0)), ctypes.byref(_weights(x=None)), None,
                                   None, None, None) == 0


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 99):
        assert isinstance(B.strerror(code), str) and B.strerror(code)


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_forward(x, x, x.view(1, 4, 8), x.view(1, 8, 4), 1)


def test_expert_load_errors(lib):
    s = _shape()
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == B.MOE_OK
    load = lib.moe_expert_load
    assert load(ctypes.byref(s), FAKE, n.value, None, None) == B.MOE_ERR_INVALID_ARG
    assert load(ctypes.byref(s), None, n.value, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert load(ctypes.byref(s), FAKE, n.value - 1, FAKE, None) == B.MOE_ERR_WORKSPACE
    assert load(ctypes.byref(s), FAKE, n.value, FAKE + 2, None) == B.MOE_ERR_ALIGNMENT
    assert load(ctypes.byref(_shape(k=0)), FAKE, n.value, FAKE, None) == B.MOE_ERR_INVALID_ARG


def test_fp8_scale_errors(lib):
    s = _shape(weight_format=1)  # 64*2/8 = 16 rows per expert: decode tiles
    assert _fwd(lib, s, _weights()) == B.MOE_ERR_INVALID_ARG  # no scales
    assert _fwd(lib, s, _weights(w_gate_up_scale=FAKE)) == B.MOE_ERR_INVALID_ARG
    sc = dict(w_gate_up_scale=FAKE, w_down_scale=FAKE + 2)
    assert _fwd(lib, s, _weights(**sc)) == B.MOE_ERR_ALIGNMENT
    s2 = _shape(weight_format=1, F_shared=64)
    sc = dict(w_gate_up_scale=FAKE, w_down_scale=FAKE, ws_gate_up=FAKE, ws_down=FAKE)
    assert _fwd(lib, s2, _weights(**sc)) == B.MOE_ERR_INVALID_ARG  # no shared scales


def test_block_m_for_e4m3_widths(lib):
    """E4M3 weights keep the 32-row tiles when a width is not a multiple of 16."""
    def bm(**kw):
        return lib.moe_block_m(ctypes.byref(_shape(**kw)))
    assert bm(T=4096, D=4096, E=8, F=14336, k=2, weight_format=1) == 256
    assert bm(T=4096, D=4096, E=8, F=14344, k=2, weight_format=1) == 32
    assert bm(T=4096, D=4104, E=8, F=14336, k=2, weight_format=1) == 32
    assert bm(T=4096, D=4096, E=8, F=14336, k=2, F_shared=8, weight_format=1) == 32
    assert bm(T=4096, D=4104, E=8, F=14336, k=2, weight_format=0) == 256
    assert bm(T=16, D=4104, E=8, F=14336, k=2, weight_format=1) == 16


def test_grads_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct moe_grads \{(.*?)\} moe_grads;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == [f[0] for f in B.Grads._fields_]


def test_backward_errors(lib):
    n = ctypes.c_size_t(0)
    size = lib.moe_backward_workspace_size
    assert size(ctypes.byref(_shape()), ctypes.byref(n)) == B.MOE_OK and n.value > 0
    assert size(ctypes.byref(_shape(weight_format=1)), ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED
    assert size(ctypes.byref(_shape(expert_begin=2, num_local_experts=4)),
                ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED
    assert size(ctypes.byref(_shape(k=0)), ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG
    size(ctypes.byref(_shape()), ctypes.byref(n))
    s = _shape()
    g = B.Grads(FAKE, FAKE, None, FAKE, FAKE, None, None)

    def bwd(shape=s, w=None, grads=g, ids=FAKE, wts=FAKE, dy=FAKE, ws=FAKE, nb=n.value):
        return lib.moe_backward(ctypes.byref(shape), ctypes.byref(w or _weights()), ids, wts, dy,
                                ctypes.byref(grads) if grads is not None else None, ws, nb, None)

    assert bwd(grads=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(grads=B.Grads(FAKE, FAKE, None, None, FAKE, None, None)) == B.MOE_ERR_INVALID_ARG
    assert bwd(dy=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(dy=FAKE + 4) == B.MOE_ERR_ALIGNMENT
    assert bwd(grads=B.Grads(FAKE, FAKE + 8, None, FAKE, FAKE, None, None)) == B.MOE_ERR_ALIGNMENT
    assert bwd(nb=n.value - 1) == B.MOE_ERR_WORKSPACE
    assert bwd(w=_weights(w_g=None)) == B.MOE_ERR_INVALID_ARG
    # a shared expert needs its two gradient outputs
    s2 = _shape(F_shared=64)
    size(ctypes.byref(s2), ctypes.byref(n))
    assert bwd(shape=s2, w=_weights(ws_gate_up=FAKE, ws_down=FAKE), nb=n.value) == B.MOE_ERR_INVALID_ARG


def test_train_entry_point_errors(lib):
    n, nt = ctypes.c_size_t(0), ctypes.c_size_t(0)
    s = _shape()
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == B.MOE_OK
    assert lib.moe_train_workspace_size(ctypes.byref(s), ctypes.byref(nt)) == B.MOE_OK
    assert nt.value > n.value  # the forward's workspace plus g | u of every row
    assert lib.moe_train_workspace_size(ctypes.byref(s), None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_train_workspace_size(ctypes.byref(_shape(weight_format=1)),
                                        ctypes.byref(nt)) == B.MOE_ERR_UNSUPPORTED
    lib.moe_train_workspace_size(ctypes.byref(s), ctypes.byref(nt))

    def fwd(shape=s, ids=FAKE, wts=FAKE, ws=FAKE, nb=nt.value):
        return lib.moe_forward_train(ctypes.byref(shape), ctypes.byref(_weights()), FAKE, ids, wts,
                                     ws, nb, None)

    assert fwd(ids=None) == B.MOE_ERR_INVALID_ARG  # the routing is needed by the backward
    assert fwd(wts=None) == B.MOE_ERR_INVALID_ARG
    assert fwd(nb=nt.value - 1) == B.MOE_ERR_WORKSPACE  # the plain forward's size is too small
    assert fwd(shape=_shape(expert_begin=2, num_local_experts=4)) == B.MOE_ERR_UNSUPPORTED
    nb = ctypes.c_size_t(0)
    lib.moe_backward_workspace_size(ctypes.byref(s), ctypes.byref(nb))
    g = B.Grads(FAKE, FAKE, None, FAKE, FAKE, None, None)

    def bwd(saved=FAKE, saved_bytes=nt.value):
        return lib.moe_backward_saved(ctypes.byref(s), ctypes.byref(_weights()), FAKE, FAKE, FAKE,
                                      ctypes.byref(g), saved, saved_bytes, FAKE, nb.value, None)

    assert bwd(saved=None) == B.MOE_ERR_INVALID_ARG
    assert bwd(saved_bytes=nt.value - 1) == B.MOE_ERR_WORKSPACE
    assert bwd(saved=FAKE + 8) == B.MOE_ERR_ALIGNMENT
