"""Benchmark: MoE layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config moe7b_bf16]

A step is one moe_forward + moe_backward over one batch of synthetic tokens
(router GEMM, route, permute, gate/up grouped GEMM with SwiGLU, down grouped
GEMM, shared experts, combine; then combine backward with the router
gradient, the four routed and four shared data/weight-gradient grouped GEMMs,
the router weight gradient and the unpermute-sum).  Inputs are resident in
HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/s; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="moe7b_bf16")
    p.add_argument("--kernel-reps", type=int, default=20, help="launches of the dominant kernel timed alone")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=2048, help="token sample for the oracle timing")
    return p.parse_args()


def cpu_baseline(cfg, inp, ntok):
    """The oracle (fp64 numpy) forward + backward on the first ntok tokens."""
    import numpy as np

    import synth
    from oracle import moe_oracle as O
    ntok = min(ntok, cfg.T)
    f = lambda a: synth.as_f64(a, cfg.dtype)  # noqa: E731
    w32 = lambda a: synth.bf16_bits_to_f32(a) if (a is not None and a.dtype == np.uint16) else a  # noqa: E731
    x = f(inp["x"][:ntok])
    dy = f(inp["dy"][:ntok])
    wgu, wd = w32(inp["w_gateup"]), w32(inp["w_down"])
    sgu, sd = f(inp["s_gateup"]), f(inp["s_down"])
    t0 = time.perf_counter()
    fw = O.forward(x, inp["w_router"], inp["bias"], wgu, wd, sgu, sd, top_k=cfg.k, score=cfg.score,
                   renorm=cfg.renorm)
    O.backward(x, inp["w_router"], wgu, wd, sgu, sd, fw, dy, score=cfg.score, renorm=cfg.renorm)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of {cfg.name}, fp64 numpy forward+backward, "
                      f"{dt:.1f} s wall, BLAS threads = all {cores} host cores"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this MoE layer build has no multi-GPU path "
              "(expert-parallel sharding is described in DESIGN.md but not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_18_amd as M
    import synth
    from mixture_experts_layer_18_amd import _lib

    _lib.load()
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    cfg = synth.CONFIG_BY_NAME[args.config]
    inp = synth.make_inputs(cfg, with_dy=True)

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    desc = M.desc_from_config(cfg)
    w = {k: dev(inp.get(k)) for k in ("w_router", "bias", "w_gateup", "w_down", "s_gateup", "s_down")}
    x = dev(inp["x"])
    dy = dev(inp["dy"])
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    saved = M.alloc_saved(desc)
    grads = M.alloc_grads(desc)
    wsf = M.alloc_workspace(desc, "forward")
    wsb = M.alloc_workspace(desc, "backward")
    stream = torch.cuda.current_stream()

    def step():
        M.moe_forward(desc, w, x, y, saved, wsf, stream)
        M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = cfg.T * args.steps / wall

    # ---- dominant kernel: the routed gate/up grouped GEMM with SwiGLU, same
    # arguments and launch configuration as inside moe_forward, timed alone
    # with events on the stream it is launched on
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
    A = T * k
    counts = saved["counts"].cpu().numpy()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    gu = lambda: M.moe_grouped_gemm("NT", "swiglu", cfg.dtype, E, A, 2 * f, d, saved["offsets"],  # noqa: E731
                                    saved["x_perm"], w["w_gateup"], saved["h"], saved["preact"], None, stream)
    dn = lambda: M.moe_grouped_gemm("NT", "none", cfg.dtype, E, A, d, f, saved["offsets"],  # noqa: E731
                                    saved["h"], w["w_down"], saved["y_perm"], None, None, stream)
    t_gu = timed(gu, args.kernel_reps)
    t_dn = timed(dn, args.kernel_reps)
    fl_gu = 2.0 * A * (2 * f) * d
    fl_dn = 2.0 * A * d * f
    ach = fl_gu / t_gu / 1e12
    fwd_tflops = (fl_gu + fl_dn) / (t_gu + t_dn) / 1e12

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights, random init)",
        "config": {
            "workload": f"{cfg.name}: MoE layer fwd+bwd, T={T} tokens (4x4096), d_model={d}, E={E} experts, "
                        f"sigmoid top-{k} + bias, expert d_ff={f}, {cfg.n_shared} shared experts d_ff="
                        f"{cfg.f_shared}",
            "tokens_per_step": T, "d_model": d, "experts": E, "top_k": k, "d_ff": f,
            "shared": f"{cfg.n_shared}x{cfg.f_shared}", "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "gate/up grouped GEMM + SwiGLU (forward, NT)",
            "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "traffic": None,
            "flop_per_launch": fl_gu, "avg_launch_us": t_gu * 1e6,
        },
        "grouped_gemm_fwd": {
            "tflops": fwd_tflops, "frac_of_peak": fwd_tflops / PEAK_BF16_TFLOPS,
            "gate_up_us": t_gu * 1e6, "down_us": t_dn * 1e6,
        },
        "loads": {"max_over_mean": float(counts.max() / counts.mean()), "empty": int((counts == 0).sum())},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
