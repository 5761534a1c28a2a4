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

Prints one JSON line.  ``value`` is tokens/s of the median step of graph
replays timed between two device synchronisations.  ``roofline`` covers the
dominant kernel: the longest stage that is one GEMM launch, among the two
GEMMs of the routed grouped FFN call and the backward's stages, timed with
the HIP events the library records on its stream after each of them
(moe_ffn_stage_events, moe_bwd_args.stage_events).  ``rooflines`` covers
every library call and ``kernel_rooflines`` every such stage.  ``train_lines`` repeats the training measurement under a
skewed expert load, ``fwd_lines`` for the forward-only workloads (8 experts
top-2, 64 experts top-8, 256 + 1 shared top-8).
``cpu_baseline`` times the CPU oracle on a bounded sample of each workload.
Progress goes to stderr.
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
    ("replay_gate", "route"), ("hash_route", "route"), ("kg_schedule", "backward"), ("kg_reduce", "backward"),
    ("shared_offsets", "backward"), ("gemm_kernel", "backward"),
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
    calls, kernels, nk = {}, {}, {}
    for d, counter, fac, key in ((fetch_dir, "FETCH_SIZE", ff, "read"), (write_dir, "WRITE_SIZE", fw, "write")):
        for (_, name), kib in per_kernel(d, counter).items():
            c = call_of(name)
            if c:
                calls.setdefault(c, {"read": 0.0, "write": 0.0})[key] += kib * 1024.0 * fac
                sn = short_name(name)
                kernels.setdefault(sn, {"read": 0.0, "write": 0.0})[key] += kib * 1024.0 * fac
                if key == "read":
                    nk[sn] = nk.get(sn, 0) + 1
    out = json.load(open(TRAFFIC)) if os.path.exists(TRAFFIC) else {}
    if out.get("source_sha") != source_hash():
        out["workloads"], out["kernels"] = {}, {}   # records of other code are dropped
    out["source_sha"] = source_hash()
    out["calibration"] = {"fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
                          "note": "bytes = counter KiB x 1024 x factor; factor = 2 GiB / counter of a plain 2 GiB copy"}
    out.setdefault("workloads", {})[workload] = {c: {k: int(v / launches) for k, v in rw.items()} for c, rw in calls.items()}
    # per kernel: bytes per launch (the average over its dispatches)
    out.setdefault("kernels", {})[workload] = {k: {kk: int(v / nk[k]) for kk, v in rw.items()}
                                               for k, rw in kernels.items() if nk.get(k)}
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
    """Per-call HBM bytes per step measured on the current kernels (None when
    the HIP code changed since the counters were taken); the per-kernel
    bytes per launch are under the key "kernels"."""
    try:
        t = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != source_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    if w is None:
        return None
    return dict(w, kernels=t.get("kernels", {}).get(workload, {}))


def summarize_counters(files):
    """Per-kernel table of rocprofv3 --pmc runs of one program (one
    counter_collection.csv per pass; a kernel_trace.csv of a pass gives the
    durations): each counter averaged over the kernel's dispatches, then
      MFMA busy  = MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs));
      clock      = GRBM_GUI_ACTIVE / 8 XCDs / average duration;
      TA busy    = TA_BUSY_avr / (GRBM_GUI_ACTIVE / 8);
      waiting    = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave cycles spent at a wait);
      L2 hit     = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum);
    and LdsUtil, LdsBankConflict, VALUBusy as rocprofv3 derives them."""
    import csv
    vals, dur = {}, {}
    for f in files:
        if f.endswith("kernel_trace.csv"):
            for r in csv.DictReader(open(f)):
                k = short_name(r["Kernel_Name"])
                dur.setdefault(k, []).append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
            continue
        for r in csv.DictReader(open(f)):
            k = short_name(r["Kernel_Name"])
            d = vals.setdefault(k, {}).setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])

    def avg(k, c):
        d = vals.get(k, {}).get(c)
        return sum(d.values()) / len(d) if d else None

    rows = []
    for k in vals:
        gui = avg(k, "GRBM_GUI_ACTIVE")
        t = sum(dur[k]) / len(dur[k]) if dur.get(k) else None
        cyc = gui / 8 if gui else None
        hit, miss = avg(k, "TCC_HIT_sum"), avg(k, "TCC_MISS_sum")
        wait, wcyc = avg(k, "SQ_WAIT_ANY"), avg(k, "SQ_WAVE_CYCLES")
        ta = avg(k, "TA_BUSY_avr")
        rows.append((k, len(next(iter(vals[k].values()))), t, avg(k, "MfmaUtil"), cyc / t / 1e9 if cyc and t else None,
                     100 * ta / cyc if ta is not None and cyc else None, avg(k, "LdsUtil"), avg(k, "LdsBankConflict"),
                     avg(k, "VALUBusy"), 100 * hit / (hit + miss) if hit is not None and miss else None,
                     100 * wait / wcyc if wait is not None and wcyc else None))
    fmt = lambda v, f: "" if v is None else format(v, f)
    print("| kernel | dispatches | avg us | MFMA busy % | clock GHz | TA busy % | LdsUtil % | LdsBankConflict | "
          "VALUBusy % | L2 hit % | waiting % |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for r in sorted(rows, key=lambda r: -(r[2] or 0)):
        if r[2] is not None and r[2] < 50e-6:
            continue
        print(f"| `{r[0][:72]}` | {r[1]} | {fmt(r[2] and r[2] * 1e6, '.1f')} | {fmt(r[3], '.1f')} | {fmt(r[4], '.2f')} | "
              f"{fmt(r[5], '.0f')} | {fmt(r[6], '.1f')} | {fmt(r[7], '.3f')} | {fmt(r[8], '.1f')} | {fmt(r[9], '.1f')} | "
              f"{fmt(r[10], '.0f')} |")


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
        # inputs dY, x (or X_perm), G|U, H, weights; outputs dx, dW; dY_perm, dG|U and dX_perm (bf16)
        # written and read once (the backward does not read Y)
        nbytes = (T * d * 2 + rows_in + A * 2 * f * 2 + A * f * 2 + 3 * E * d * f * 2
                  + T * d * 4 + 3 * E * d * f * 4 + 2 * (A * d * 2 + A * 2 * f * 2 + A * d * 2))
        out["backward"] = (12.0 * A * d * f + 4.0 * A * d, nbytes, PEAK_BF16_TFLOPS)
    return out


def blas_info():
    """BLAS library, version and thread count numpy uses (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"library": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads")}
    except Exception:  # pragma: no cover
        pass
    return {"library": None, "version": None, "threads": None}


def host_cores():
    return len(os.sched_getaffinity(0))


ONE_CORE_SNIPPET = r"""
import json, os, sys, time
os.sched_setaffinity(0, {min(os.sched_getaffinity(0))})
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle
from workloads import CONFIGS, make_inputs
cfg = CONFIGS["tiny"]
inp = make_inputs(cfg)
n, t0 = 0, time.perf_counter()
while time.perf_counter() - t0 < 3.0:
    oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], cfg.k, cfg.score, False,
                   sel_bias=inp["bias"])
    n += 1
dt = time.perf_counter() - t0
res = {"value": round(n * cfg.T / dt, 1), "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "calls": n}
from oracle import pure
L = lambda a: np.asarray(a, np.float64).tolist()
args = [L(inp[key]) for key in ("x", "w_router", "w_gate_up", "w_down")]
bias = L(inp["bias"])
n, t0 = 0, time.perf_counter()
while time.perf_counter() - t0 < 3.0:
    pure.forward(*args, cfg.k, cfg.score, False, sel_bias=bias)
    n += 1
dt = time.perf_counter() - t0
res["pure_python"] = {"value": round(n * cfg.T / dt, 1), "unit": "tokens/s", "cores": 1, "calls": n}
print(json.dumps(res))
"""


def oracle_one_core():
    """The oracle's forward on the tiny fp32 workload (T=64, 8 experts top-2)
    on one host core with single-threaded BLAS, and the same forward in plain
    Python loops (oracle/pure.py), in a child process started before this
    process touches the GPU."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", ONE_CORE_SNIPPET, ROOT], env=env, capture_output=True, text=True,
                           timeout=120)
        out = json.loads(r.stdout.strip().splitlines()[-1])
        out.update(kind="oracle", sample="tiny workload (T=64 d=32 E=8 top-2 fp32) forward, repeated for 3 s, "
                                         "one core, BLAS single-threaded")
        out["pure_python"].update(kind="oracle (oracle/pure.py)",
                                  sample="the same forward in plain Python loops, repeated for 3 s, one core")
        return out
    except Exception as e:  # pragma: no cover
        return {"error": str(e)[:200]}


def cpu_baseline(cfg, inp, train, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the workload."""
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
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": host_cores(), "blas": blas_info(),
            "kind": "oracle",
            "sample": f"first {tokens} of {cfg.T} tokens of the same workload, "
                      f"{'forward+backward' if train else 'forward'} in fp64 numpy ({dt:.1f} s)"}


def routing_stats(cfg, inp, idx_gpu, counts_gpu):
    """Expert load of the first forward (max and min over mean of the counts)
    and, from the oracle's fp64 router on every token, the tokens excluded as
    near-ties (k-th and (k+1)-th keys within 1e-6 relative) and the tokens
    outside them whose expert set differs from the GPU's (expected 0)."""
    import numpy as np
    import oracle
    c = np.asarray(counts_gpu, np.float64)
    mean = c.mean()
    r = oracle.route(inp["x"], inp["w_router"], cfg.k, cfg.score, inp["bias"], inp["logit_offset"])
    excl = r["margin"] < 1e-6
    g = np.sort(np.asarray(idx_gpu, np.int64), axis=1)
    o = np.sort(r["idx"], axis=1)
    mism = int((np.any(g != o, axis=1) & ~excl).sum())
    return {"load_max_over_mean": round(float(c.max() / mean), 3), "load_min_over_mean": round(float(c.min() / mean), 3),
            "near_tie_excluded": int(excl.sum()), "idx_mismatch_outside_near_ties": mism}


def time_replays(graph, steps, warmup):
    """Graph replays: `warmup` untimed, then exactly `steps` timed between
    two device synchronisations.  Events on the replay stream around every
    replay give per-step times; returns (median ms, mean ms of the events,
    wall-clock ms per step)."""
    import statistics
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        graph.replay()
    ev[steps].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return statistics.median(per), sum(per) / steps, wall


def stage_algorithmic(cfg):
    """Per stage of the routed grouped FFN call (moe_ffn_stage) and of the
    backward (moe_bwd_stage): (flops, bytes, peak TFLOP/s or None for a
    memory-bound stage) -- each tensor read or written once."""
    T, d, E, k, f, A = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.T * cfg.k
    fs = cfg.f_shared * cfg.shared
    return {
        # x rows and W_gate_up in; H out, and G|U out in training
        "ffn_up": (4.0 * A * d * f, T * d * 2 + E * 2 * f * d * 2 + A * f * 2 + (A * 2 * f * 2 if cfg.train else 0),
                   PEAK_BF16_TFLOPS),
        # H and W_down in, Y_perm (fp32) out
        "ffn_down": (2.0 * A * d * f, A * f * 2 + E * d * f * 2 + A * d * 4, PEAK_BF16_TFLOPS),
        # dy rows in, dY_perm = bf16(g dy) and each row's gate out
        "combine": (0, T * d * 2 + A * d * 2 + A * 4 + T * k * 12, None),
        # gate backward (dg partials in) and the router weight gradient
        "router": (2.0 * A * d, A * (f // 32) * 4 + T * d * 2 + A * 4 + E * d * 4 + T * k * 12, None),
        # dy rows and W_down in; G|U and H in for the epilogue; dG|dU and the dg partials out
        "dgrad_down": (2.0 * A * d * f, T * d * 2 + E * d * f * 2 + A * 2 * f * 2 + A * f * 2 + A * 2 * f * 2
                       + A * (f // 32) * 4, PEAK_BF16_TFLOPS),
        "wgrad_down": (2.0 * A * d * f, A * d * 2 + A * f * 2 + E * d * f * 4, PEAK_BF16_TFLOPS),
        "wgrad_up": (4.0 * A * d * f, A * 2 * f * 2 + T * d * 2 + E * 2 * f * d * 4, PEAK_BF16_TFLOPS),
        "dgrad_up": (4.0 * A * d * f, A * 2 * f * 2 + E * 2 * f * d * 2 + A * d * 2, PEAK_BF16_TFLOPS),
        "shared": (12.0 * T * d * fs, 0, PEAK_BF16_TFLOPS),
        # bf16 dX_perm rows and W_r rows in, dx (fp32) out
        "unpermute": (0, A * d * 2 + T * d * 4 + E * d * 4 + T * k * 12, None),
    }


# kernel of each stage that dominates it (for the per-kernel roofline and its
# PMC traffic record)
STAGE_KERNEL = {
    "ffn_up": "gemm_kernel<256, 256, true, true, false, 0, false>",
    "ffn_down": "gemm_kernel<256, 256, true, true, false, 1, false>",
    "dgrad_down": "gemm_kernel<256, 256, true, false, false, 2, false>",
    "wgrad_down": "gemm_kernel<256, 256, false, false, true, 1, false>",
    "wgrad_up": "gemm_kernel<256, 256, false, false, true, 1, true>",
    "dgrad_up": "gemm_kernel<256, 256, true, false, false, 3, false>",
    "unpermute": "unpermute_bwd_lds_kernel<8>",
}


def dominant_roofline(line):
    """The roofline entry of a measured line's dominant kernel: the longest
    stage that is one GEMM kernel (the routed grouped FFN's two, the
    backward's), else the longest library call."""
    kr = {k: v for k, v in line.get("kernel_rooflines", {}).items() if "kernel" in v}
    if kr:
        dom = max(kr, key=lambda k: kr[k]["ms"])
        roof = dict(kr[dom])
        where = f"grouped FFN stage {dom[4:]}" if dom.startswith("ffn_") else f"moe_backward stage {dom}"
        roof["kernel"] = f"{roof['kernel']} ({where}, one launch per step)"
        return roof
    dom = max(line["rooflines"], key=lambda c: line["rooflines"][c]["ms"])
    roof = dict(line["rooflines"][dom])
    roof["kernel"] = f"moe_{dom} (library call, all of its kernels)"
    return roof


def roofline_entry(flops, nbytes, peak_flops, ms, traffic=None):
    t = ms * 1e-3
    if flops and peak_flops and (not nbytes or flops / nbytes >= peak_flops / PEAK_HBM_GBS * 1e3):
        ach = flops / t / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(ach / peak_flops, 4), "ms": round(ms, 4), "flops": flops, "bytes": nbytes,
                "peak_dtype": "fp32" if peak_flops < PEAK_BF16_TFLOPS else "bf16", "traffic": traffic}
    ach = nbytes / t / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "ms": round(ms, 4), "flops": flops, "bytes": nbytes,
            "peak_dtype": None, "traffic": traffic}


def build_layer(cfg, inp, device, fuse=True, packed=False):
    """packed: a forward-only layer packs its expert weights once, at
    construction (outside any timed region), as a serving layer would."""
    import torch
    from mixture_experts_layer_free_amd.layer import MoELayer, Shape
    d = lambda k: _dev(inp.get(k), device)
    shape = Shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, torch.bfloat16, cfg.score, cfg.shared, cfg.f_shared,
                  cfg.bias_update, cfg.gamma, cfg.train, fuse_permute=fuse,
                  packed_weights=packed and not cfg.train and cfg.f % 128 == 0)
    layer = MoELayer(shape, d("w_router"), d("w_gate_up"), d("w_down"), d("bias"), d("logit_offset"),
                     d("w_gate_up_shared"), d("w_down_shared"), device=device)
    return layer, d("x"), (d("dy") if cfg.train else None)


def measure(cfg, a, device, fuse=True, cpu_tokens=None, graph=True):
    """One workload: tokens/s from graph replays (median step), per-call and
    per-backward-stage times from an eager timed region with HIP events on
    the calls' stream, routing statistics of the first forward, and the
    oracle on a bounded sample."""
    import statistics
    import numpy as np
    import torch
    from mixture_experts_layer_free_amd import _lib
    from mixture_experts_layer_free_amd.layer import CallTimer
    train = cfg.train
    inp = None
    log(f"[bench] {cfg.name}: generating inputs")
    from workloads import make_inputs
    inp = make_inputs(cfg)
    layer, x, dy = build_layer(cfg, inp, device, fuse, packed=not a.given_weights)

    def step(timer=None, stage_events=None):
        layer.forward(x, timer=timer)
        if train:
            layer.backward(x, dy, timer=timer, stage_events=stage_events)

    # first forward: the routing under the initial bias
    layer.forward(x)
    torch.cuda.synchronize()
    idx0 = layer.idx.cpu().numpy()
    counts0 = layer.counts.cpu().numpy()
    if train:
        layer.backward(x, dy)
    log(f"[bench] {cfg.name}: warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # eager timed region: events around every library call, after each GEMM
    # of the routed grouped FFN call, and after every backward stage
    timer = CallTimer()
    nst, nfs = len(_lib.BWD_STAGES), len(_lib.FFN_STAGES)
    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(a.steps)]
    ffn_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nfs + 1)] for _ in range(a.steps)]
    for evs in stage_ev + ffn_ev:
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        layer.forward(x, timer=timer, ffn_events=ffn_ev[i])
        if train:
            stage_ev[i][0].record()
            layer.backward(x, dy, timer=timer, stage_events=stage_ev[i][1:])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / a.steps * 1e3
    calls = {n: round(statistics.median(ea.elapsed_time(eb) for ea, eb in timer.pairs[n]), 4) for n in timer.pairs}
    fstages = {"ffn_" + name: round(statistics.median(ffn_ev[i][si].elapsed_time(ffn_ev[i][si + 1])
                                                      for i in range(a.steps)), 4)
               for si, name in enumerate(_lib.FFN_STAGES)}
    stages = {}
    if train:
        for si, name in enumerate(_lib.BWD_STAGES):
            stages[name] = round(statistics.median(stage_ev[i][si].elapsed_time(stage_ev[i][si + 1])
                                                   for i in range(a.steps)), 4)
    log(f"[bench] {cfg.name}: eager {eager_ms:.3f} ms/step; calls {calls}; grouped FFN stages {fstages}; "
        f"backward stages {stages}")
    if graph:
        g = layer.capture(x, dy)
        log(f"[bench] {cfg.name}: timing {a.steps} graph replays")
        med, mean, wall = time_replays(g, a.steps, a.warmup)
        del g
    else:
        med = mean = wall = eager_ms
    log(f"[bench] {cfg.name}: {med:.4f} ms/step (median), mean {mean:.4f}, wall {wall:.4f}")
    traffic = measured_traffic(cfg.name)
    ktraffic = (traffic or {}).get("kernels", {})
    rooflines = {}
    for call, (flops, nbytes, peak_flops) in algorithmic(cfg, fuse, fuse).items():
        if call in calls:
            tr = traffic.get(call) if traffic else None
            rooflines[call] = roofline_entry(flops, nbytes, peak_flops, calls[call],
                                             (tr["read"] + tr["write"]) if tr else None)
    kernels = {}
    timed = {**fstages, **stages}
    for name, (flops, nbytes, peak_flops) in stage_algorithmic(cfg).items():
        if name in timed and (flops or nbytes):
            kn = STAGE_KERNEL.get(name)
            tr = ktraffic.get(kn) if kn else None
            kernels[name] = roofline_entry(flops, nbytes, peak_flops, timed[name],
                                           (tr["read"] + tr["write"]) if tr else None)
            if kn:
                kernels[name]["kernel"] = kn
    res = {"ms_per_step": round(med, 4), "ms_per_step_mean": round(mean, 4), "ms_per_step_wall": round(wall, 4),
           "tokens_per_s": round(cfg.T / (med * 1e-3), 1), "eager_ms_per_step": round(eager_ms, 4),
           "calls_ms": calls, "rooflines": rooflines,
           "expert_tflops": round(expert_flops(cfg, train) / (med * 1e-3) / 1e12, 1)}
    res["grouped_ffn_stages_ms"] = fstages
    res["kernel_rooflines"] = kernels
    if train:
        res["backward_stages_ms"] = stages
    res["routing"] = routing_stats(cfg, inp, idx0, counts0)
    log(f"[bench] {cfg.name}: routing {res['routing']}")
    del layer, x, dy
    torch.cuda.empty_cache()
    if cpu_tokens:
        log(f"[bench] {cfg.name}: cpu oracle on {cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, train, cpu_tokens)
    del inp
    return res


# hipBLASLt (torch.mm) GEMMs with the M, N, K of the six expert GEMMs of the
# training step, each dense over all A = T*k rows (the weight gradients as
# one product with K = A): the same flops as the grouped kernels, bf16 out.
LIB_GEMMS = ("up", "down", "dgrad_down", "wgrad_down", "wgrad_up", "dgrad_up")


def library_gemms(cfg, steps, device):
    import torch
    A, d, f = cfg.T * cfg.k, cfg.d, cfg.f
    g = torch.Generator(device=device).manual_seed(0)
    r = lambda *s: (torch.randn(*s, device=device, generator=g) * 0.5).to(torch.bfloat16)
    X, Wgu, Wd = r(A, d), r(2 * f, d), r(d, f)
    Hh, dYp, dGU = r(A, f), r(A, d), r(A, 2 * f)
    ops = {
        "up": lambda: torch.mm(X, Wgu.t()),            # [A,d] x [d,2f]
        "down": lambda: torch.mm(Hh, Wd.t()),          # [A,f] x [f,d]
        "dgrad_down": lambda: torch.mm(dYp, Wd),       # [A,d] x [d,f]
        "wgrad_down": lambda: torch.mm(dYp.t(), Hh),   # [d,A] x [A,f]
        "wgrad_up": lambda: torch.mm(dGU.t(), X),      # [2f,A] x [A,d]
        "dgrad_up": lambda: torch.mm(dGU, Wgu),        # [A,2f] x [2f,d]
    }
    flops = {"up": 4.0 * A * d * f, "down": 2.0 * A * d * f, "dgrad_down": 2.0 * A * d * f,
             "wgrad_down": 2.0 * A * d * f, "wgrad_up": 4.0 * A * d * f, "dgrad_up": 4.0 * A * d * f}
    out = {}
    for name in LIB_GEMMS:
        fn = ops[name]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[name] = {"ms": round(ms, 4), "tflops": round(flops[name] / (ms * 1e-3) / 1e12, 1)}
        log(f"[bench] hipBLASLt {name}: {ms:.4f} ms, {out[name]['tflops']} TFLOP/s")
    return out


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
    if not a.given_weights:
        pgu, pd = _lib.moe_pack_expert_weights(wgu, wd)
        del wgu, wd
        run = lambda: _lib.moe_grouped_ffn_packed(xs, None, g_off, pgu, pd, cfg.f, h=h, y=y)
    else:
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
                                  f"{rows} rows; grouped FFN only, no all-to-all"
                                  + ("" if a.given_weights else "; expert weights packed in tile order once"),
                      "global_batch": cfg.T, "seq_len": None, "parallelism": "ep8 (one rank's share on 1 GPU)"},
           "expert_tflops": round(ach, 1), "roofline": roof}
    print(json.dumps(res), flush=True)


CPU_TOKENS = {"train": 16384, "train_skew": 16384, "fine": 4096, "coarse": 512, "dsv3": 16}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train",
                    choices=["train", "train_skew", "fine", "coarse", "dsv3", "dsv3_ep8"])
    ap.add_argument("--fwd-lines", default="fine,coarse,dsv3",
                    help="forward-only workloads measured after the training line (comma-separated; '' for none)")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="oracle sample size of the headline (tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--no-fwd", action="store_true", help="skip the forward-only lines")
    ap.add_argument("--given-weights", action="store_true",
                    help="forward-only layers use the expert weights as given (default: packed in tile order "
                         "once, at construction, as a serving layer would)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="also time hipBLASLt GEMMs with the M, N, K of the training step's six expert GEMMs")
    ap.add_argument("--no-fuse-permute", action="store_true",
                    help="the permute copies X_perm, and the up-projection and W_gate_up's weight gradient read it, "
                         "instead of gathering x rows through token_of")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs of this bench into profiles/traffic.json")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "STEPS"),
                    help="print a rocprofv3 kernel_stats.csv of this bench as a markdown table")
    ap.add_argument("--summarize-counters", nargs="+", metavar="COUNTER_CSV",
                    help="print rocprofv3 --pmc counter_collection.csv files (one per pass) as a per-kernel table")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 2 GiB device-to-device copy (HBM reference and PMC byte calibration)")
    a = ap.parse_args()
    if a.summarize_stats:
        summarize_stats(a.summarize_stats[0], int(a.summarize_stats[1]), a.workload)
        return
    if a.summarize_pmc:
        # the profiled run is `bench.py --no-graph --no-fwd --no-cpu-baseline` with the same --steps/--warmup
        # (plus one first forward/backward before the warm-up)
        summarize_pmc(*a.summarize_pmc, workload=a.workload, launches=a.steps + a.warmup + 1)
        return
    if a.summarize_counters:
        summarize_counters(a.summarize_counters)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this layer's hot path runs on a single MI355X and has no multi-GPU "
              f"mode (asked for --gpus {a.gpus}).", file=sys.stderr)
        sys.exit(2)
    # the one-core oracle runs in a child process, started before this
    # process touches the GPU
    one_core = None
    if not a.no_cpu_baseline and a.workload == "train" and not a.copy_probe:
        log("[bench] oracle on one core (tiny workload)")
        one_core = oracle_one_core()

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
        res = {"copy_bytes_per_launch": 2 * n, "ms": round(ms, 4), "gb_per_s": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        # reference read-only and write-only streams of the same 2 GiB (torch's own kernels)
        f32 = src.view(torch.float32)
        for name, fn in (("read", lambda: f32.sum()), ("write", lambda: dst.fill_(3))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(a.steps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            t = ev[0].elapsed_time(ev[1]) / a.steps
            res[f"{name}_gb_per_s"] = round(n / (t * 1e-3) / 1e9, 1)
        print(json.dumps(res), flush=True)
        return
    from workloads import EP_SHARDS
    if a.workload in EP_SHARDS:
        bench_ep_shard(a)
        return
    from mixture_experts_layer_free_amd import _lib
    from workloads import CONFIGS

    _lib.lib()
    cfg = CONFIGS[a.workload]
    train = cfg.train
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    fuse = not a.no_fuse_permute
    cpu_tokens = None if a.no_cpu_baseline else (a.cpu_tokens or CPU_TOKENS[cfg.name])
    head = measure(cfg, a, device, fuse, cpu_tokens, graph=not a.no_graph)
    lib_gemms = library_gemms(cfg, a.steps, device) if (a.library_gemms and train) else None
    train_lines = {}
    if train and not a.no_fwd and cfg.name == "train":
        c = CONFIGS["train_skew"]
        r = measure(c, a, device, fuse, None, graph=not a.no_graph)
        r["workload"] = describe(c, True) + " with the Zipf logit offset of the 64-expert forward (skewed load)"
        train_lines["train_skew"] = r
    fwd_lines = {}
    if train and not a.no_fwd:
        for name in [n for n in a.fwd_lines.split(",") if n]:
            c = CONFIGS[name]
            r = measure(c, a, device, True, None if a.no_cpu_baseline else CPU_TOKENS[name], graph=not a.no_graph)
            r["workload"] = describe(c, False) + ", permute fused into the expert GEMM" + (
                "" if a.given_weights else ", expert weights packed in tile order once at construction")
            fwd_lines[name] = r
    roof = dominant_roofline(head)
    res = {"metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": describe(cfg, train) + (", permute fused into the expert GEMMs" if fuse else "")
                      + ("" if train or a.given_weights else ", expert weights packed in tile order once at construction"),
                      "global_batch": cfg.T, "seq_len": None, "parallelism": "none (1 GPU)"},
           "step_mode": ("eager" if a.no_graph else "hip_graph_replay") + ", ms_per_step = median of the steps",
           "roofline": roof}
    for k in ("ms_per_step_mean", "ms_per_step_wall", "eager_ms_per_step", "calls_ms", "grouped_ffn_stages_ms",
              "backward_stages_ms",
              "expert_tflops", "rooflines", "kernel_rooflines", "routing"):
        if k in head:
            res[k] = head[k]
    if train_lines:
        res["train_lines"] = train_lines
    if fwd_lines:
        res["fwd_lines"] = fwd_lines
    if lib_gemms:
        res["library_gemms"] = lib_gemms
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
        if one_core:
            res["cpu_baseline"]["one_core_tiny"] = one_core
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
