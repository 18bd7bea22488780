"""Dense float64 evaluation of the MoE layer, for tiny inputs only.

An independent check of the oracle: it is vectorised instead of looping, runs
every expert on every token (E times the needed work) and zeroes the
unselected ones through a dense gate matrix, as the glossary "MoE (Mixture of
Experts - Mezcla de Expertos)", section 3 step 2, describes the unselected
scores being cancelled.  Library routines stand in for the hand-written loops:
numpy matmul for every contraction, a stable numpy argsort for the top-k,
scipy's softmax and expit for the normalisation and the SiLU.
"""
import numpy as np
import scipy.special as sps
import torch


def f64(t):
    return None if t is None else t.to(torch.float64).numpy()


def weights64(t, scale):
    """Expert weights as float64: bf16 widened, or E4M3 codes decoded by
    torch's float8_e4m3fn type (a library decode) times each row's scale."""
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale.double().numpy()[..., None]
    return f64(t)


def dense_logits(inp):
    """fp32 logits; a bias in the logits is added before the rounding, a
    selection-only bias is not added at all."""
    X = f64(inp.x)
    l = X @ f64(inp.w_g).T
    if inp.router_bias is not None and not inp.shape.bias_select:
        l = l + inp.router_bias.to(torch.float64).numpy()[None, :]
    # the selection is defined on fp32 logits
    return l.astype(np.float32).astype(np.float64)


def dense_routing(inp):
    """Top-k by stable argsort of the selection keys, softmax of the logits.
    With a selection-only bias the keys are the fp32 sum logit + bias."""
    l = dense_logits(inp)
    key = l
    if inp.router_bias is not None and inp.shape.bias_select:
        b = inp.router_bias.numpy().astype(np.float32)
        key = (l.astype(np.float32) + b[None, :]).astype(np.float64)
    k = inp.shape.k
    ids = np.argsort(-key, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(l, ids, axis=1)
    p = sps.softmax(chosen, axis=1)
    return ids, p, l


def swiglu_ffn(X, w_gu, w_dn):
    """Textbook SwiGLU FFN: W_down (SiLU(W_a x) * (W_b x)), W_a = first half."""
    F = w_gu.shape[0] // 2
    g = X @ w_gu[:F].T
    u = X @ w_gu[F:].T
    h = g * sps.expit(g) * u
    return h @ w_dn.T


def dense_forward(inp):
    s = inp.shape
    ids, p, _ = dense_routing(inp)
    X = f64(inp.x)
    T = X.shape[0]
    G = np.zeros((T, s.E))
    np.put_along_axis(G, ids, p, axis=1)
    Wgu = weights64(inp.w_gate_up, inp.w_gate_up_scale)
    Wd = weights64(inp.w_down, inp.w_down_scale)
    Y = np.zeros((T, s.D))
    for e in range(s.E):
        Y += G[:, e:e + 1] * swiglu_ffn(X, Wgu[e], Wd[e])
    if s.Fs:
        Y += swiglu_ffn(X, weights64(inp.ws_gate_up, inp.ws_gate_up_scale),
                        weights64(inp.ws_down, inp.ws_down_scale))
    return Y, ids, p
