#!/usr/bin/env python3
"""Throughput of the token-choice MoE layer on one MI355X.

One step = one pass of the layer's hot path over one batch of synthetic,
seeded input already resident in HBM:
  * workload "train" (default): 64 experts top-8, T=16384, d_model=2048,
    expert width 1024, sqrt(softplus) router: route -> permute -> grouped
    SwiGLU experts -> combine -> bias update -> backward (fwd+bwd);
  * workload "fine": 64 experts top-8, T=8192, sigmoid router with a Zipf
    logit offset: forward + bias update;
  * "coarse" (8 experts top-2) and "dsv3" (256+1 shared, top-8) forwards.

Prints one JSON line (rank 0).  ``roofline`` covers the dominant library
call, timed with HIP events on its stream inside the timed region;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (fwd; fwd+bwd) at E=64,k=8 on 1 GPU; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev(a, device):
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def describe(cfg, train):
    sh = f" + {cfg.shared} shared (f={cfg.f_shared})" if cfg.shared else ""
    return (f"{cfg.name}: T={cfg.T} d_model={cfg.d} E={cfg.E}{sh} top-{cfg.k} expert_ffn={cfg.f} "
            f"{cfg.score} router fp32, bf16 experts, {'fwd+bwd' if train else 'fwd'}"
            f"{' + bias update' if cfg.bias_update else ''}")


def expert_flops(cfg, train):
    A = cfg.T * cfg.k
    f = 6 * A * cfg.d * cfg.f + 6 * cfg.T * cfg.d * cfg.f_shared * cfg.shared
    if train:
        f += 12 * A * cfg.d * cfg.f
    return f


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(cfg, inp, train, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the workload."""
    import numpy as np
    import oracle
    sl = slice(0, tokens)
    x = inp["x"][sl]
    t0 = time.perf_counter()
    fwd = oracle.forward(x, inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score, True,
                         sel_bias=inp["bias"], logit_offset=inp["logit_offset"],
                         w_gate_up_shared=inp.get("w_gate_up_shared"), w_down_shared=inp.get("w_down_shared"))
    if cfg.bias_update:
        oracle.bias_update(inp["bias"], fwd["counts"], tokens, cfg.k, cfg.gamma)
    if train:
        oracle.backward(fwd, inp["dy"][sl], x, inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.score, True)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {tokens} of {cfg.T} tokens of the same workload, "
                      f"{'forward+backward' if train else 'forward'} in fp64 numpy ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train", choices=["train", "fine", "coarse", "dsv3"])
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle sample size (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 2 GiB device-to-device copy (HBM reference and PMC byte calibration)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this layer's hot path runs on a single MI355X and has no multi-GPU "
              f"mode (asked for --gpus {a.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if a.copy_probe:
        n = 1 << 31
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(a.steps):
            dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / a.steps
        print(json.dumps({"copy_bytes_per_launch": 2 * n, "ms": round(ms, 4),
                          "gb_per_s": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return
    from mixture_experts_layer_free_amd import _lib
    from mixture_experts_layer_free_amd.layer import CallTimer, MoELayer, Shape
    from workloads import CONFIGS, make_inputs

    _lib.lib()
    cfg = CONFIGS[a.workload]
    train = cfg.train
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"[bench] generating inputs for {cfg.name}")
    inp = make_inputs(cfg)
    d = lambda k: _dev(inp.get(k), device)
    shape = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, cfg.shared, cfg.f_shared,
                  cfg.bias_update, cfg.gamma, train)
    layer = MoELayer(shape, d("w_router"), d("w_gate_up"), d("w_down"), d("bias"), d("logit_offset"),
                     d("w_gate_up_shared"), d("w_down_shared"), device=device)
    x = d("x")
    dy = d("dy") if train else None

    def step(timer=None):
        layer.forward(x, timer=timer)
        if train:
            layer.backward(x, dy, timer=timer)

    log(f"[bench] warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # timed region 1: eager launches with HIP events around every library call
    timer = CallTimer()
    log(f"[bench] timing {a.steps} eager steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(timer)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / a.steps * 1e3
    calls = {n: round(timer.mean_ms(n), 4) for n in timer.pairs}
    log(f"[bench] eager {eager_ms:.3f} ms/step, per call ms: {calls}")
    # timed region 2: the same step captured once in a HIP graph and replayed
    if a.no_graph:
        ms = eager_ms
    else:
        graph = layer.capture(x, dy)
        for _ in range(a.warmup):
            graph.replay()
        torch.cuda.synchronize()
        log(f"[bench] timing {a.steps} graph replays")
        t0 = time.perf_counter()
        for _ in range(a.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / a.steps * 1e3
        log(f"[bench] graph {ms:.3f} ms/step")
    value = cfg.T / (ms * 1e-3)

    # dominant call: the routed grouped FFN (forward) or the backward
    A = cfg.T * cfg.k
    dom = "backward" if train else "grouped_ffn"
    if dom == "grouped_ffn":
        flops = 6 * A * cfg.d * cfg.f
    else:
        flops = 12 * A * cfg.d * cfg.f
    dom_ms = calls.get(dom, float("nan"))
    achieved = flops / (dom_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": f"moe_{dom} ({'12' if train else '6'}*A*d*f flops per call)",
            "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None, "call_ms": dom_ms}

    res = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": describe(cfg, train), "global_batch": cfg.T, "seq_len": None,
                      "parallelism": "none (1 GPU)"},
           "eager_ms_per_step": round(eager_ms, 4), "step_mode": "eager" if a.no_graph else "hip_graph_replay",
           "calls_ms": calls, "expert_tflops": round(expert_flops(cfg, train) / (ms * 1e-3) / 1e12, 1),
           "roofline": roof}
    if not a.no_cpu_baseline:
        tokens = a.cpu_tokens or (1024 if train else cfg.T)
        log(f"[bench] cpu oracle on {tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, train, tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
