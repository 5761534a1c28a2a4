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
import re
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


CSRC = os.path.join(ROOT, "mixture_experts_layer_free_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _code_only(text):
    """Source text without comments and with whitespace runs collapsed: an
    edit that changes no code leaves it unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash():
    """sha256 over the code of the HIP sources (comments and layout left out):
    measured HBM traffic is only reported for the kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(_code_only(open(os.path.join(CSRC, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


# which library call launched a kernel (by kernel name), for per-call PMC sums
CALL_OF = [
    ("router_logits", "route"), ("topk_gate_kernel", "route"),
    ("perm_", "permute"),
    ("gemm_kernel<256, 256, true, true, false", "grouped_ffn"), ("gemm_kernel<128, 128, true, true, false", "grouped_ffn"),
    ("ffn_up_f32", "grouped_ffn"), ("ffn_down_f32", "grouped_ffn"),
    ("combine_kernel", "combine"), ("bias_update_kernel", "bias_update"),
    ("combine_bwd", "backward"), ("gate_bwd", "backward"), ("router_wgrad", "backward"), ("unpermute_bwd", "backward"),
    ("router_seg_schedule", "backward"), ("aux_dl_dense", "backward"), ("router_dense_wgrad", "backward"),
    ("fill_zero", "backward"), ("aux_prob", "aux_loss"), ("aux_loss_final", "aux_loss"),
    ("replay_gate", "route"), ("hash_route", "route"),
    ("gemm_kernel", "backward"),
]


def call_of(name):
    for pat, call in CALL_OF:
        if pat in name:
            return call
    return None


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload, launches):
    """Per-call HBM bytes per step from rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (KiB per dispatch), each scaled by what the counter reads for the
    plain 2 GiB copy of --copy-probe; merged into profiles/traffic.json."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        tot = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                tot.setdefault((r["Dispatch_Id"], r["Kernel_Name"]), 0.0)
                tot[(r["Dispatch_Id"], r["Kernel_Name"])] += float(r["Counter_Value"])
        return tot

    def copy_factor(d, counter, known):
        vals = [v for (_, name), v in per_kernel(d, counter).items() if "copy" in name.lower()]
        if not vals:
            raise SystemExit(f"no copy kernel in the {counter} run under {d}")
        return known / (sum(vals) / len(vals) * 1024.0)

    n = 1 << 31
    ff = copy_factor(copy_fetch_dir, "FETCH_SIZE", n)
    fw = copy_factor(copy_write_dir, "WRITE_SIZE", n)
    calls = {}
    for d, counter, fac, key in ((fetch_dir, "FETCH_SIZE", ff, "read"), (write_dir, "WRITE_SIZE", fw, "write")):
        for (_, name), kib in per_kernel(d, counter).items():
            c = call_of(name)
            if c:
                calls.setdefault(c, {"read": 0.0, "write": 0.0})[key] += kib * 1024.0 * fac
    out = json.load(open(TRAFFIC)) if os.path.exists(TRAFFIC) else {}
    out["source_sha"] = source_hash()
    out["calibration"] = {"fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
                          "note": "bytes = counter KiB x 1024 x factor; factor = 2 GiB / counter of a plain 2 GiB copy"}
    out.setdefault("workloads", {})[workload] = {c: {k: int(v / launches) for k, v in rw.items()} for c, rw in calls.items()}
    os.makedirs(os.path.dirname(TRAFFIC), exist_ok=True)
    json.dump(out, open(TRAFFIC, "w"), indent=1)
    print(json.dumps(out["workloads"][workload]))


def short_name(name):
    n = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("moe_gemm::", "")
    return n[:n.index("(")] if "(" in n else n


def summarize_stats(stats_csv, steps, title):
    """Markdown table of a rocprofv3 --stats kernel summary: per kernel the
    launches, average duration and the library call it belongs to, then the
    per-step time of each call (sum of its kernels), comparable to the
    event-timed calls_ms of the bench line."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"### {title}", "", "| kernel | call | launches | avg us | min us | max us | % |",
             "|---|---|---:|---:|---:|---:|---:|"]
    per_call = {}
    for r in rows:
        c = call_of(r["Name"]) or "-"
        lines.append(f"| `{short_name(r['Name'])}` | {c} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
        if c != "-":
            per_call[c] = per_call.get(c, 0.0) + float(r["TotalDurationNs"]) / steps / 1e6
    lines += ["", f"Per step ({steps} steps in the run), sum of each call's kernels, ms:", ""]
    lines += [f"- {c}: {v:.4f}" for c, v in per_call.items()]
    print("\n".join(lines))


def measured_traffic(workload):
    try:
        t = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def algorithmic(cfg, fused=False, gather=None):
    """Per library call: (flops, bytes, peak TFLOP/s of its arithmetic) that
    the method itself needs -- every tensor read or written once, weights
    once, intermediates written once and read once.  fused: the permute moves
    indices only (no X_perm).  gather (default: fused): the up-projection
    (and in training W_gate_up's weight gradient) reads its rows from x
    through token_of, not from X_perm."""
    gather = fused if gather is None else gather
    T, d, E, k, f, A = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.T * cfg.k
    xb = 2 if cfg.dtype == "bf16" else 4
    gu = A * 2 * f * 2 if cfg.train else 0                  # saved G|U (training)
    rows_in = T * d * xb if gather else A * d * xb          # the up-projection's input rows
    out = {
        "route": (2.0 * T * d * E, T * d * xb + E * d * 4 + T * E * 4 + T * k * 8, 157.3),
        "permute": (0, (0 if fused else T * d * xb + A * d * xb) + T * k * 8 + A * 4, None),
        "grouped_ffn": (6.0 * A * d * f, rows_in + 3 * E * d * f * xb + 2 * A * f * xb + A * d * 4 + gu,
                        PEAK_BF16_TFLOPS),
        "combine": (0, A * d * 4 + T * d * 4 * (2 if cfg.shared else 1) + T * k * 8, None),
        "bias_update": (0, E * 12, None),
    }
    if cfg.shared:
        fs = cfg.f_shared
        out["shared_ffn"] = (6.0 * T * d * fs, T * d * xb + 3 * d * fs * xb + 2 * T * fs * xb + T * d * 4,
                             PEAK_BF16_TFLOPS)
    if cfg.train:
        # inputs dY, Y, x (or X_perm), G|U, H, weights; outputs dx, dW; dY_perm, dG|U, dX_perm written and
        # read once
        nbytes = (T * d * 2 + A * d * 4 + rows_in + A * 2 * f * 2 + A * f * 2 + 3 * E * d * f * 2
                  + T * d * 4 + 3 * E * d * f * 4 + 2 * (A * d * 2 + A * 2 * f * 2 + A * d * 4))
        out["backward"] = (12.0 * A * d * f + 4.0 * A * d, nbytes, PEAK_BF16_TFLOPS)
    return out


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


def fwd_line(_lib, a, device):
    """Forward-only tokens/s on the 64-expert top-8 shape (T=8192, sigmoid
    router with the Zipf-skewed logit offset, bias update), graph replays."""
    import torch
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    from workloads import CONFIGS, make_inputs
    cfg = CONFIGS["fine"]
    log(f"[bench] forward line: generating inputs for {cfg.name}")
    inp = make_inputs(cfg)
    d = lambda k: _dev(inp.get(k), device)
    layer = MoELayer(Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, 0, 0, cfg.bias_update,
                           cfg.gamma, False), d("w_router"), d("w_gate_up"), d("w_down"), d("bias"),
                     d("logit_offset"), device=device)
    x = d("x")
    for _ in range(a.warmup):
        layer.forward(x)
    graph = layer.capture(x)
    for _ in range(a.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / a.steps * 1e3
    log(f"[bench] forward line: {ms:.3f} ms/step")
    return {"workload": describe(cfg, False) + ", permute fused into the expert GEMM",
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "ms_per_step": round(ms, 4), "expert_tflops": round(expert_flops(cfg, False) / (ms * 1e-3) / 1e12, 1)}


def bench_ep_shard(a):
    """The grouped expert FFN on one expert-parallel rank's share: the global
    batch is routed and permuted over all experts, and the rank's contiguous
    expert block (its rows of X_perm and its experts' weights) goes through
    moe_grouped_ffn, timed with HIP events on its stream.  The all-to-all
    exchange around it is not part of this measurement."""
    import torch
    from mixture_experts_layer_free_amd import _lib
    from workloads import ep_shard, expert_weight_range, make_inputs

    _lib.lib()
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    cfg, e0, e1 = ep_shard(a.workload)
    log(f"[bench] {a.workload}: routing {cfg.T} tokens over {cfg.E} experts; rank experts {e0}..{e1 - 1}")
    inp = make_inputs(cfg, experts=False)
    x = _dev(inp["x"], device)
    idx, _, _ = _lib.moe_route(x, _dev(inp["w_router"], device), cfg.k, cfg.score, sel_bias=_dev(inp["bias"], device))
    _, offsets, _, _, x_perm = _lib.moe_permute(idx, x, cfg.E)
    off = offsets[e0:e1 + 1].cpu().numpy().astype("int64")
    rows = int(off[-1] - off[0])
    xs = x_perm[int(off[0]):int(off[-1])]
    g_off = torch.from_numpy((off - off[0]).astype("int32")).to(device)
    del x, x_perm
    log(f"[bench] {rows} rows for {e1 - e0} experts (min {int((off[1:] - off[:-1]).min())}, "
        f"max {int((off[1:] - off[:-1]).max())}); generating their weights")
    wgu_np, wd_np = expert_weight_range(cfg, e0, e1)
    wgu, wd = _dev(wgu_np, device), _dev(wd_np, device)
    del wgu_np, wd_np
    h = torch.empty((rows, cfg.f), dtype=torch.bfloat16, device=device)
    y = torch.empty((rows, cfg.d), dtype=torch.float32, device=device)
    run = lambda: _lib.moe_grouped_ffn(xs, g_off, wgu, wd, h=h, y=y)
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(a.steps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / a.steps
    G, d, f = e1 - e0, cfg.d, cfg.f
    flops = 6.0 * rows * d * f
    nbytes = rows * d * 2 + 3 * G * d * f * 2 + 2 * rows * f * 2 + rows * d * 4
    ach = flops / (ms * 1e-3) / 1e12
    bound = "mfma" if flops / nbytes >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3 else "hbm"
    roof = ({"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / PEAK_BF16_TFLOPS, 4)} if bound == "mfma" else
            {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
    roof.update({"kernel": "moe_grouped_ffn (library call, all of its kernels)", "call_ms": round(ms, 4),
                 "flops": flops, "bytes": nbytes, "traffic": None})
    res = {"metric": "expert FFN rows/s of one expert-parallel rank's share", "value": round(rows / (ms * 1e-3), 1),
           "unit": "rows/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{a.workload}: rank 0 of 8 on the 256-expert top-8 shape (d_model={d}, "
                                  f"expert_ffn={f}): experts {e0}..{e1 - 1} of a {cfg.T}-token global batch, "
                                  f"{rows} rows; grouped FFN only, no all-to-all",
                      "global_batch": cfg.T, "seq_len": None, "parallelism": "ep8 (one rank's share on 1 GPU)"},
           "expert_tflops": round(ach, 1), "roofline": roof}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train", choices=["train", "fine", "coarse", "dsv3", "dsv3_ep8"])
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle sample size (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--no-fwd", action="store_true", help="skip the forward-only line on the 64-expert shape")
    ap.add_argument("--no-fuse-permute", action="store_true",
                    help="the permute copies X_perm, and the up-projection and W_gate_up's weight gradient read it, "
                         "instead of gathering x rows through token_of")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs of this bench into profiles/traffic.json")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "STEPS"),
                    help="print a rocprofv3 kernel_stats.csv of this bench as a markdown table")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 2 GiB device-to-device copy (HBM reference and PMC byte calibration)")
    a = ap.parse_args()
    if a.summarize_stats:
        summarize_stats(a.summarize_stats[0], int(a.summarize_stats[1]), a.workload)
        return
    if a.summarize_pmc:
        # the profiled run is `bench.py --no-graph --no-fwd --no-cpu-baseline` with the same --steps/--warmup
        summarize_pmc(*a.summarize_pmc, workload=a.workload, launches=a.steps + a.warmup)
        return
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
    from workloads import EP_SHARDS
    if a.workload in EP_SHARDS:
        bench_ep_shard(a)
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
                  cfg.bias_update, cfg.gamma, train, fuse_permute=not a.no_fuse_permute)
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

    # per-call rooflines: algorithmic work per call / the call's event time
    traffic = measured_traffic(cfg.name)
    rooflines = {}
    gather = not a.no_fuse_permute                 # the expert GEMMs read x through token_of
    fused = gather                                 # and then no X_perm is written
    for call, (flops, nbytes, peak_flops) in algorithmic(cfg, fused, gather).items():
        if call not in calls:
            continue
        t = calls[call] * 1e-3
        tr = traffic.get(call) if traffic else None
        if flops and flops / nbytes >= peak_flops / PEAK_HBM_GBS * 1e3:   # at or above the ridge: compute-bound
            ach, peak, unit = flops / t / 1e12, peak_flops, "TFLOP/s"
            bound, dt = "mfma", ("fp32" if peak_flops < PEAK_BF16_TFLOPS else "bf16")
        else:
            ach, peak, unit, bound, dt = nbytes / t / 1e9, PEAK_HBM_GBS, "GB/s", "hbm", None
        rooflines[call] = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                           "frac": round(ach / peak, 4), "call_ms": calls[call], "peak_dtype": dt,
                           "flops": flops, "bytes": nbytes, "traffic": (tr["read"] + tr["write"]) if tr else None}
    dom = max((c for c in rooflines), key=lambda c: calls[c])
    roof = dict(rooflines[dom])
    roof["kernel"] = f"moe_{dom} (library call, all of its kernels)"

    res = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": describe(cfg, train) + (", permute fused into the expert GEMMs"
                                                          if fused else ""),
                      "global_batch": cfg.T, "seq_len": None,
                      "parallelism": "none (1 GPU)"},
           "eager_ms_per_step": round(eager_ms, 4), "step_mode": "eager" if a.no_graph else "hip_graph_replay",
           "calls_ms": calls, "expert_tflops": round(expert_flops(cfg, train) / (ms * 1e-3) / 1e12, 1),
           "roofline": roof, "rooflines": rooflines}
    if train and not a.no_fwd:
        res["fwd"] = fwd_line(_lib, a, device)
    if not a.no_cpu_baseline:
        # about 10-30 s of oracle work on the host's cores
        tokens = a.cpu_tokens or {"train": 16384, "fine": 8192, "coarse": 4096, "dsv3": 1024}[cfg.name]
        log(f"[bench] cpu oracle on {tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, train, tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
