"""The parity bars of the GPU tests and CPU emulations of the roundings the
GPU path makes, from which tests/test_tolerances.py derives each bar.

Test infrastructure: float64 numpy, with bf16 rounding through torch's
round-to-nearest-even conversion.  Nothing here calls the GPU library or
shares code with it.

Bars:
  Y_TOL          max|y - y_oracle| <= Y_TOL * RMS(y_oracle) (forward layer)
  MARGIN         a token whose oracle top-k margin exceeds MARGIN must pick
                 the oracle's expert set; the routing weights of a matching
                 set agree within WEIGHT_TOL
  SHARD_SUM_TOL  expert-parallel shards' y add up to the whole layer's y
                 within SHARD_SUM_TOL * RMS(y)
  KSPLIT_TOL     two kernel families that group the K sum differently
                 (E4M3 vs bf16 weights) agree within KSPLIT_TOL * RMS(y)
  GRAD_RMS_TOL, GRAD_MAX_TOL
                 per gradient tensor, RMS(g - g0) and max|g - g0| over the
                 scale of g0 (grad_error)
"""
import numpy as np
import torch

Y_TOL = 2e-2
MARGIN = 1e-4
WEIGHT_TOL = 1e-4
SHARD_SUM_TOL = 1e-2
KSPLIT_TOL = 1e-2
GRAD_RMS_TOL = 1e-2
GRAD_MAX_TOL = 1.5e-1


def bf16(a):
    """Round to bf16 (nearest even) through fp32, returned as float64."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


def f64(t):
    return t.float().numpy().astype(np.float64)


def grad_error(g, g0, scale=0.0):
    """(RMS error, max error), both relative to max(RMS(g0), scale)."""
    g = np.asarray(g, np.float64)
    rms = max(float(np.sqrt(np.mean(g0 * g0))), scale, 1e-30)
    return float(np.sqrt(np.mean((g - g0) ** 2))) / rms, float(np.max(np.abs(g - g0))) / rms


def bias_terms_scale(dp, ids, p, E):
    """RMS over experts of the root-sum-square of d_bias's terms dl[t, j].

    d_bias[e] sums dl over the slots routed to e; the terms have either sign
    and can cancel far below their own size, while each carries its own
    rounding, so the terms' size is the scale its error is measured on."""
    dl = p * (dp - (p * dp).sum(1, keepdims=True))
    ss = np.zeros(E)
    np.add.at(ss, np.asarray(ids).ravel(), (dl * dl).ravel())
    return float(np.sqrt(np.mean(ss)))


def fp32_dot(X, W, pieces=1, chunk=16):
    """X @ W.T (W is [m, K], K contiguous, as the weights are stored) summed
    the way the GPU's MFMA tiles sum it: K is cut into `pieces` contiguous
    ranges (the K-split of a GEMM's last round, or the waves of a router
    tile), each summed chunk by chunk with one fp32 rounding per chunk of
    `chunk` products (an MFMA adds its products to the fp32 accumulator), and
    the pieces' fp32 sums added in order."""
    K = X.shape[1]
    nc = -(-K // chunk)
    bounds = [int(round(i * nc / pieces)) for i in range(pieces + 1)]
    tot = None
    for q in range(pieces):
        acc = np.zeros((X.shape[0], W.shape[0]), np.float32)
        for c in range(bounds[q], bounds[q + 1]):
            k0, k1 = c * chunk, min(K, (c + 1) * chunk)
            # the chunk's products summed exactly (float64), then one fp32 rounding
            acc = (acc.astype(np.float64) + X[:, k0:k1] @ W[:, k0:k1].T).astype(np.float32)
        tot = acc if tot is None else (tot.astype(np.float64) + acc).astype(np.float32)
    return tot.astype(np.float64)


def _silu(g):
    return g / (1.0 + np.exp(-g))


def emulate_forward(inp, ids, p, pieces=None, chunk=16, w_gate_up=None, w_down=None):
    """y of the layer's experts with the GPU path's one rounding that matters:
    h = bf16(SiLU(g) * u) is stored in bf16 between the two GEMMs.  With
    `pieces` None, g and u are exact; else they are summed as fp32_dot(pieces,
    chunk).  Everything after h is exact.  Expert weights default to inp's
    bf16 tensors (pass callables e -> float64 array for other weights).
    Returns (y, {group: (rows, h)}) with the shared expert as group E."""
    s = inp.shape
    x = f64(inp.x)
    wgu = w_gate_up or (lambda e: f64(inp.w_gate_up[e]))
    wd = w_down or (lambda e: f64(inp.w_down[e]))
    T = x.shape[0]
    y = np.zeros((T, s.D))
    hs = {}

    def run(ts, pw, Wgu, Wd, F):
        X = x[ts]
        if pieces is None:
            g, u = X @ Wgu[:F].T, X @ Wgu[F:].T
        else:
            g, u = fp32_dot(X, Wgu[:F], pieces, chunk), fp32_dot(X, Wgu[F:], pieces, chunk)
        h = bf16(_silu(g) * u)
        y[ts] += pw[:, None] * (h @ Wd.T)
        return h

    for e in range(s.E):
        ts, js = np.nonzero(ids == e)
        if ts.size:
            hs[e] = (ts, run(ts, p[ts, js], wgu(e), wd(e), s.F))
    if s.Fs:
        hs[s.E] = (np.arange(T), run(np.arange(T), np.ones(T), f64(inp.ws_gate_up),
                                     f64(inp.ws_down), s.Fs))
    return y, hs


def emulate_backward(inp, ids, p, dy, mistake=None):
    """The backward pass with the GPU path's bf16 roundings and exact sums.

    Per expert and routed row: dh' = W_down^T bf16(dy) (dy enters its GEMM as
    bf16); h = bf16(SiLU(g) u); dp = <dh', h>; dg = bf16(p dh' u SiLU'(g)),
    du = bf16(p dh' SiLU(g)) (stored bf16 for the next GEMMs); dx rows =
    [dg du] W_gate_up; dW_down = sum_rows bf16(p dy) h^T; dW_gate_up =
    sum_rows [dg du] x^T.  Router: dl = p (dp - sum_j p dp), dW_g[e] = sum dl x,
    d_bias[e] = sum dl (bias in the logits only), dx += sum_j dl W_g[ids].
    x and every weight are bf16 already; g and u keep fp32 precision, whose
    error is 2^16 times below bf16's, so they are exact here.

    `mistake` plants one error, to show the bars catch it: "dsilu" drops the
    g(1 - sigmoid) term of SiLU', "dl_sign" flips the softmax-centering sign,
    "dw_down_p" leaves p out of dW_down.  Returns oracle.backward's keys."""
    s = inp.shape
    T, k = ids.shape
    x, wg = f64(inp.x), f64(inp.w_g)
    dy = np.asarray(dy, np.float64)
    dyb = bf16(dy)
    out = dict(dx=np.zeros((T, s.D)), dw_g=np.zeros((s.E, s.D)), d_bias=np.zeros(s.E),
               dw_gate_up=np.zeros((s.E, 2 * s.F, s.D)), dw_down=np.zeros((s.E, s.D, s.F)))
    dp = np.zeros((T, k))

    def expert(ts, pw, Wgu, Wd, F):
        X = x[ts]
        g, u = X @ Wgu[:F].T, X @ Wgu[F:].T
        sig = 1.0 / (1.0 + np.exp(-g))
        sl = g * sig
        h = bf16(sl * u)
        dhp = dyb[ts] @ Wd
        dh = pw[:, None] * dhp
        dsilu = sig if mistake == "dsilu" else sig * (1.0 + g * (1.0 - sig))
        dgu = np.concatenate([bf16(dh * u * dsilu), bf16(dh * sl)], 1)
        pdy = dy[ts] if mistake == "dw_down_p" else pw[:, None] * dy[ts]
        return (dhp * h).sum(1), dgu @ Wgu, bf16(pdy).T @ h, dgu.T @ X

    for e in range(s.E):
        ts, js = np.nonzero(ids == e)
        if ts.size == 0:
            continue
        dp[ts, js], dxr, out["dw_down"][e], out["dw_gate_up"][e] = expert(
            ts, p[ts, js], f64(inp.w_gate_up[e]), f64(inp.w_down[e]), s.F)
        np.add.at(out["dx"], ts, dxr)
    if s.Fs:
        ts = np.arange(T)
        _, dxr, out["dws_down"], out["dws_gate_up"] = expert(
            ts, np.ones(T), f64(inp.ws_gate_up), f64(inp.ws_down), s.Fs)
        out["dx"] += dxr
    centre = (p * dp).sum(1, keepdims=True)
    dl = p * (dp + centre) if mistake == "dl_sign" else p * (dp - centre)
    for e in range(s.E):
        ts, js = np.nonzero(ids == e)
        out["dw_g"][e] = (dl[ts, js][:, None] * x[ts]).sum(0)
        if inp.router_bias is not None and not s.bias_select:
            out["d_bias"][e] = dl[ts, js].sum()
    for j in range(k):
        out["dx"] += dl[:, j:j + 1] * wg[ids[:, j]]
    out["dp"] = dp
    return out
