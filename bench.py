"""Benchmark of one sparse-MoE SwiGLU layer forward pass on one MI355X.

A step is one full ``moe_forward`` call (router, grouping, gate/up GEMM with
SwiGLU, down GEMM, combine) over one batch of synthetic tokens already resident
in HBM.  Default workload: the Mixtral-8x7B-shaped prefill layer
(T=4096, D=4096, E=8, top-2, d_ff=14336).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; % bf16 MFMA peak (prefill), % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNELS = ("moe_router", "moe_align", "moe_gemm_gate_up", "moe_gemm_down", "moe_combine")
LLC_BYTES = 256 << 20       # MI355X Infinity Cache


def _log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def _kernel_sources_sha(gemm_file):
    """sha256 over the sources that make up the gate/up kernel."""
    h = hashlib.sha256()
    for f in (gemm_file, "device.hpp", "launch.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_mixture_experts_prefix_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic_from_profile(workload, T, sha):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    PMC summary, or None when there is none or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "gemm_gate_up_%s_T%d_pmc.md" % (workload, T))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b:
        return None
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def _cpu_baseline(inp, target_s):
    """The CPU oracle (router + experts per token) on the first n tokens."""
    import oracle
    import workloads as W

    s = inp.shape

    def run(n):
        sub = dataclasses.replace(inp, shape=s.with_T(n), x=inp.x[:n].contiguous())
        t0 = time.perf_counter()
        oracle.forward(sub)
        return time.perf_counter() - t0

    cores = oracle.num_threads()
    n0 = max(1, min(s.T, cores))
    t_cal = run(n0)
    n = int(max(n0, min(s.T, n0 * target_s / max(t_cal, 1e-6))))
    t = run(n) if n != n0 else t_cal
    return {"value": n / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d tokens of the %s workload, router + top-%d experts%s per token, "
                      "%.1f s wall" % (n, s.T, "same", s.k, " + shared expert" if s.Fs else "", t)}


def _bench_backward(args, s, wl, g, moe, torch, W, dev):
    """Backward pass timing: gradients of sum <dy, y> for the routing of one
    forward call, on the same inputs; dy ~ N(0, 1) fp32.  --saved: that call is
    the training forward and the backward reads its saved g | u."""
    if s.fp8 or args.ep != 1:
        raise SystemExit("--backward takes bf16 weights and the whole layer")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    wts = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    saved = None
    if args.saved:
        _, _, _, saved = moe.moe_forward_train(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, g.router_bias,
                                               g.ws_gate_up, g.ws_down, bias_select=s.bias_select,
                                               topk_ids=ids, topk_w=wts)
    else:
        moe.moe_forward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, g.router_bias, g.ws_gate_up,
                        g.ws_down, topk_ids=ids, topk_w=wts, bias_select=s.bias_select)
    dy = W.normal_f32((s.T, s.D), 0, 99, 1.0).to(dev)
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, s.Fs, moe.bias_mode(g.router_bias, s.bias_select))
    ws = torch.empty(moe.backward_workspace_size(shape), dtype=torch.uint8, device=dev)
    grads = moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, ids, wts, dy, g.router_bias,
                             g.ws_gate_up, g.ws_down, bias_select=s.bias_select, workspace=ws,
                             saved=saved)

    def step():
        moe.moe_backward(g.x, g.w_g, g.w_gate_up, g.w_down, s.k, ids, wts, dy, g.router_bias,
                         g.ws_gate_up, g.ws_down, bias_select=s.bias_select, workspace=ws, grads=grads,
                         saved=saved)

    def timed(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t

    timed(step, args.warmup)
    elapsed = timed(step, args.steps)
    ms = elapsed / args.steps * 1e3
    _log("timed %d backward steps: %.3f ms/step" % (args.steps, ms))
    forward_ms = {}
    if args.saved:  # the price of keeping g | u: the two forwards, timed apart from the backward
        y = torch.empty((s.T, s.D), dtype=torch.float32, device=dev)
        fws = torch.empty(moe.train_workspace_size(shape), dtype=torch.uint8, device=dev)
        common = (g.x, g.w_g, g.w_gate_up, g.w_down, s.k, g.router_bias, g.ws_gate_up, g.ws_down)
        kw = dict(bias_select=s.bias_select, y=y, topk_ids=ids, topk_w=wts, workspace=fws)
        for name, fn in (("forward", lambda: moe.moe_forward(*common, **kw)),
                         ("forward_train", lambda: moe.moe_forward_train(*common, **kw))):
            timed(fn, args.warmup)
            forward_ms[name] = round(timed(fn, args.steps) / args.steps * 1e3, 4)
        _log("forward %.3f ms, training forward %.3f ms" % (forward_ms["forward"],
                                                            forward_ms["forward_train"]))
    # algorithmic work: dgrad and wgrad of the three expert products (6 each
    # per routed row and unit of D*F, likewise for the shared expert) and the
    # router's two products; the recomputation of g and u is not counted
    rows = s.T * s.k
    flops = 12 * rows * s.D * s.F + 12 * s.T * s.D * s.Fs + 4 * s.T * s.D * s.E
    achieved = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "MoE-layer backward tokens/s",
        "value": round(s.T * args.steps / elapsed, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based normal draws: x ~ N(0,1), weights ~ N(0,0.02), "
                "dy ~ N(0,1), bf16 weights)",
        "config": {"workload": wl.name, "pass": "backward (saved g|u)" if args.saved else "backward",
                   "T": s.T, "D": s.D, "E": s.E, "k": s.k,
                   "d_ff": s.F, "shared_d_ff": s.Fs, "router_bias": bool(s.router_bias)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "kernel": "moe_backward_saved (whole call)" if args.saved else
                               "moe_backward (whole call)", "traffic": None},
        "cpu_baseline": None,
    }
    if forward_ms:
        out["forward_ms"] = forward_ms
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--T", type=int, default=None, help="token count override (decode sweeps)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (removes host launch gaps)")
    ap.add_argument("--ep", type=int, default=1,
                    help="expert-parallel degree: time the shard of one rank (E/ep experts; the "
                         "shared expert on rank 0) at the workload's real shape")
    ap.add_argument("--rank", type=int, default=0, help="which shard --ep times")
    ap.add_argument("--fp8", action="store_true",
                    help="expert weights as E4M3 codes with one fp32 scale per row (the same "
                         "draws quantised per row)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (moe_backward) for the routing of one forward "
                         "call instead of the forward pass")
    ap.add_argument("--saved", action="store_true",
                    help="with --backward: take the routing and g | u from moe_forward_train")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="run one plain device copy of this many GiB first (a known-size kernel "
                         "for calibrating rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path; --ep/--rank "
              "time one expert-parallel rank's shard on one GPU (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from sparse_mixture_experts_prefix_amd import build as native

    if not os.path.exists(native.LIB_PATH):
        native.build()
    import sparse_mixture_experts_prefix_amd as moe

    moe.load_library()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")

    wl = W.WORKLOADS[args.workload]
    s = wl.shape if args.T is None else wl.shape.with_T(args.T)
    if args.fp8:
        s = dataclasses.replace(s, fp8=True)
    if args.ep < 1 or s.E % args.ep or not 0 <= args.rank < args.ep:
        raise SystemExit("--ep must divide E=%d and 0 <= --rank < --ep" % s.E)
    _log("generating %s T=%d inputs" % (wl.name, s.T))
    inp = W.make_inputs(s, seed=0)
    e_loc = s.E // args.ep
    e0 = args.rank * e_loc
    if args.ep > 1:  # this rank's shard: its experts, the shared expert on rank 0 only
        keep_shared = args.rank == 0
        def cut(t):
            return None if t is None else t[e0:e0 + e_loc].contiguous()

        def sh(t):
            return t if keep_shared else None

        inp = dataclasses.replace(inp, w_gate_up=cut(inp.w_gate_up), w_down=cut(inp.w_down),
                                  w_gate_up_scale=cut(inp.w_gate_up_scale),
                                  w_down_scale=cut(inp.w_down_scale), ws_gate_up=sh(inp.ws_gate_up),
                                  ws_down=sh(inp.ws_down), ws_gate_up_scale=sh(inp.ws_gate_up_scale),
                                  ws_down_scale=sh(inp.ws_down_scale))
    g = inp.to(dev)
    shard = dict(expert_begin=e0) if args.ep > 1 else {}
    fs_used = s.Fs if (args.ep == 1 or args.rank == 0) else 0
    # Rotate over weight copies when one copy would sit in the Infinity Cache.
    wel = 1 if s.fp8 else 2  # bytes per expert weight
    wbytes = (inp.w_gate_up.numel() + inp.w_down.numel()) * wel
    n_copies = 1 if wbytes > 4 * LLC_BYTES else 4
    sets = [g]

    def clone(t):
        return None if t is None else t.clone()

    for _ in range(n_copies - 1):
        sets.append(dataclasses.replace(
            g, w_gate_up=clone(g.w_gate_up), w_down=clone(g.w_down), ws_gate_up=clone(g.ws_gate_up),
            ws_down=clone(g.ws_down), w_gate_up_scale=clone(g.w_gate_up_scale),
            w_down_scale=clone(g.w_down_scale), ws_gate_up_scale=clone(g.ws_gate_up_scale),
            ws_down_scale=clone(g.ws_down_scale)))

    def scales(q):
        return ((q.w_gate_up_scale, q.w_down_scale, q.ws_gate_up_scale, q.ws_down_scale)
                if s.fp8 else None)

    fmt = moe.WEIGHTS_FP8_E4M3 if s.fp8 else moe.WEIGHTS_BF16
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, fs_used, s.router_bias,
                           e0 if args.ep > 1 else 0, e_loc if args.ep > 1 else 0, fmt)
    ws = moe.alloc_workspace(shape, dev)
    y = torch.empty((s.T, s.D), dtype=torch.float32, device=dev)
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    wts = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)

    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        _log("copy calibration: %d bytes read, %d bytes written" % (n, n))

    if args.backward:
        _bench_backward(args, s, wl, g, moe, torch, W, dev)
        return

    def step(i):
        q = sets[i % len(sets)]
        moe.moe_forward(q.x, q.w_g, q.w_gate_up, q.w_down, s.k, q.router_bias, q.ws_gate_up,
                        q.ws_down, y=y, topk_ids=ids, topk_w=wts, workspace=ws, scales=scales(q),
                        **shard)

    run = step
    if args.graph:
        for i in range(2 * len(sets)):  # compile-time state (kernel attributes) before capture
            step(i)
        torch.cuda.synchronize()
        graphs = []
        for i in range(len(sets)):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(i)
            graphs.append(gr)
        torch.cuda.synchronize()

        def run(i):
            graphs[i % len(graphs)].replay()

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    _log("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step))

    # Per-kernel durations from HIP events recorded on the launch stream.
    ev = [moe.HipEvents(6) for _ in range(args.steps)]
    for i in range(args.steps):
        q = sets[i % len(sets)]
        moe.moe_forward_timed(ev[i], q.x, q.w_g, q.w_gate_up, q.w_down, s.k, q.router_bias,
                              q.ws_gate_up, q.ws_down, y=y, topk_ids=ids, topk_w=wts, workspace=ws,
                              scales=scales(q), **shard)
    torch.cuda.synchronize()
    per_kernel = {name: float(np.mean([e.elapsed_ms(j, j + 1) for e in ev]))
                  for j, name in enumerate(KERNELS)}
    for e in ev:
        e.close()

    loads = np.bincount(ids.cpu().numpy().ravel(), minlength=s.E)
    local = loads[e0:e0 + e_loc]  # the whole layer when ep == 1
    touched = int((local > 0).sum())
    n_assign = int(local.sum())   # routed rows this call computes
    # algorithmic work of this call: router over all E, its routed rows, the
    # shared expert where it runs; bytes: touched experts' weights (with their
    # row scales when E4M3), W_g, x, y
    gu_flops = 4 * n_assign * s.D * s.F + 4 * s.T * s.D * fs_used
    flops = 2 * s.T * s.D * s.E + gu_flops + 2 * n_assign * s.D * s.F + 2 * s.T * s.D * fs_used
    sc = 4 if s.fp8 else 0  # scale bytes per weight row
    nbytes = (touched * (W.expert_params(s) * wel + (2 * s.F + s.D) * sc)
              + 3 * s.D * fs_used * wel + (2 * fs_used + s.D) * sc * (fs_used > 0)
              + s.E * s.D * 2 + s.T * s.D * 2 + s.T * s.D * 4)
    t_ideal = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
    layer_bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9) else "hbm"

    gu_ms = per_kernel["moe_gemm_gate_up"]
    shape = moe.make_shape(s.T, s.D, s.E, s.F, s.k, s.Fs, s.router_bias, weight_format=fmt)
    gemm_file = "gemm_prefill.hip" if moe.moe_block_m(shape) == 256 else "gemm_decode.hip"
    wl_tag = wl.name + ("_fp8" if s.fp8 else "")
    traffic = _traffic_from_profile(wl_tag, s.T, _kernel_sources_sha(gemm_file)) if args.ep == 1 else None
    if layer_bound == "mfma":
        achieved = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        # expert weights of the gate/up half actually touched (+ row scales) + gathered x
        gu_bytes = (touched * 2 * s.F * (s.D * wel + sc) + 2 * fs_used * (s.D * wel + sc)
                    + s.T * s.D * 2)
        achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = "moe_gemm_gate_up"
    roof["kernel_ms"] = round(gu_ms, 4)
    roof["traffic"] = traffic

    out = {
        "metric": METRIC,
        "value": round(s.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based normal draws: x ~ N(0,1), weights ~ N(0,0.02), bf16"
                + ("; expert weights quantised per row to e4m3)" if s.fp8 else ")"),
        "config": {"workload": wl.name, "T": s.T, "D": s.D, "E": s.E, "k": s.k, "d_ff": s.F,
                   "shared_d_ff": s.Fs, "router_bias": bool(s.router_bias),
                   "expert_weights": "e4m3 + fp32 row scale" if s.fp8 else "bf16",
                   "weight_copies_rotated": n_copies, "hip_graph": bool(args.graph),
                   **({"expert_parallel": args.ep, "rank": args.rank, "local_experts": [e0, e0 + e_loc],
                       "local_rows": n_assign} if args.ep > 1 else {})},
        "roofline": roof,
        "layer": {"bound": layer_bound, "algorithmic_tflop": round(flops / 1e12, 4),
                  "algorithmic_gb": round(nbytes / 1e9, 4), "ideal_ms": round(t_ideal * 1e3, 4),
                  "frac": round(t_ideal * 1e3 / ms_per_step, 4),
                  "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
                  "touched_experts": touched, "max_expert_rows": int(loads.max())},
        "kernel_ms": {k_: round(v, 4) for k_, v in per_kernel.items()},
    }
    if not args.no_cpu_baseline and args.ep == 1:
        _log("timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = _cpu_baseline(inp, args.cpu_seconds)
        out["cpu_baseline"]["sample"] = out["cpu_baseline"]["sample"].replace("same", wl.name)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
