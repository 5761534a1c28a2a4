"""The benchmark's host-side arithmetic (no GPU needed): per-stage work,
roofline classification, the choice of the dominant kernel, and the one-GPU
rule of the command line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def test_stage_work_adds_up_to_the_step_and_calls():
    """The six expert GEMMs of the stages carry the step's expert flops
    (routed, no shared expert), and the two grouped FFN stages the flops of
    the grouped FFN call."""
    cfg = CONFIGS["train"]
    st = bench.stage_algorithmic(cfg)
    gemms = ("ffn_up", "ffn_down", "dgrad_down", "wgrad_down", "wgrad_up", "dgrad_up")
    assert sum(st[g][0] for g in gemms) == bench.expert_flops(cfg, True)
    calls = bench.algorithmic(cfg, True, True)
    assert st["ffn_up"][0] + st["ffn_down"][0] == calls["grouped_ffn"][0]
    A, d, f = cfg.T * cfg.k, cfg.d, cfg.f
    assert st["ffn_up"][0] == st["wgrad_up"][0] == st["dgrad_up"][0] == 4.0 * A * d * f
    assert st["ffn_down"][0] == st["wgrad_down"][0] == st["dgrad_down"][0] == 2.0 * A * d * f
    # the training forward writes G|U for the backward, the forward-only layer does not
    fwd = bench.stage_algorithmic(CONFIGS["fine"])
    c2 = CONFIGS["fine"]
    assert fwd["ffn_up"][1] == c2.T * c2.d * 2 + c2.E * 2 * c2.f * c2.d * 2 + c2.T * c2.k * c2.f * 2


def test_roofline_bound_follows_the_ridge():
    peak = bench.PEAK_BF16_TFLOPS
    ridge = peak * 1e12 / (bench.PEAK_HBM_GBS * 1e9)   # flop per byte
    above = bench.roofline_entry(ridge * 1e9 * 1.01, 1e9, peak, 1.0)
    below = bench.roofline_entry(ridge * 1e9 * 0.99, 1e9, peak, 1.0)
    assert above["bound"] == "mfma" and below["bound"] == "hbm"
    # 1e12 flops in 1 ms = 1000 TFLOP/s = 0.4 of 2.5 PFLOP/s; 4e9 bytes in 1 ms = 4 TB/s = 0.5 of 8 TB/s
    assert above["unit"] == "TFLOP/s" and bench.roofline_entry(1e12, 1e6, peak, 1.0)["frac"] == 0.4
    hb = bench.roofline_entry(0, 4e9, None, 1.0)
    assert hb["bound"] == "hbm" and hb["achieved"] == 4000.0 and hb["frac"] == 0.5


def test_dominant_kernel_is_the_longest_gemm_stage():
    def entry(ms, kernel=None):
        e = bench.roofline_entry(1e12, 1e6, bench.PEAK_BF16_TFLOPS, ms)
        if kernel:
            e["kernel"] = kernel
        return e
    line = {"kernel_rooflines": {"ffn_up": entry(1.10, "K_up"), "wgrad_up": entry(1.09, "K_wu"),
                                 "unpermute": entry(5.0)},   # no single kernel: never the dominant one
            "rooflines": {"backward": entry(4.0)}}
    r = bench.dominant_roofline(line)
    assert r["kernel"] == "K_up (grouped FFN stage up, one launch per step)" and r["ms"] == 1.1
    line["kernel_rooflines"]["wgrad_up"] = entry(1.2, "K_wu")
    assert bench.dominant_roofline(line)["kernel"] == "K_wu (moe_backward stage wgrad_up, one launch per step)"
    # no stage timed: the longest library call
    r = bench.dominant_roofline({"rooflines": {"combine": entry(0.2), "grouped_ffn": entry(1.7)}})
    assert r["kernel"] == "moe_grouped_ffn (library call, all of its kernels)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
