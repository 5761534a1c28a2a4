"""Seeded synthetic inputs for the token-choice MoE layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It draws random numbers and stores them; it holds none of the
layer's arithmetic (no routing, no scoring, no expert math).

Workloads (shapes, distributions and seeds) follow the five configurations the
MoE layer is measured on:

* ``tiny``   T=64, d_model=32, 8 SwiGLU experts of width 64, top-2, fp32,
              softmax over the chosen raw logits, selection bias U(-0.05, 0.05),
              weights N(0, 0.02), x N(0, 1), seed 0.  ``tiny_dense`` is the
              1-expert, k=1 variant of the same shapes.
* ``coarse`` T=4096, d_model=4096, 8 experts of width 14336, top-2, bf16,
              softmax over the chosen, no bias, seed 1.
* ``fine``   T=8192, d_model=2048, 64 experts of width 1024, top-8, bf16,
              sigmoid normalised over the chosen, a per-expert logit offset
              0.5*ln(r^-1.2) for a random Zipf rank r (skewed load), bias 0
              then +-1e-3 per step, seed 2.
* ``dsv3``   T=4096, d_model=7168, 256 routed experts of width 2048 plus one
              shared expert of width 2048, top-8, bf16, sigmoid normalised,
              weights N(0, 0.006), bias U(-0.05, 0.05), seed 3.
* ``train``  the fine-grained shape at T=16384 with sqrt(softplus) scores,
              forward plus backward with dY N(0, 1) in bf16, seed 4.
              ``train_skew`` adds the Zipf logit offset of ``fine`` (skewed
              expert load in training).

One expert-parallel rank's share (``ep_shard``): ``dsv3_ep8`` is rank 0 of 8
ranks on the ``dsv3`` shape.  The global batch is 8 x 4096 tokens drawn like
``dsv3``'s (same seed and distributions, T = 32768), routed over all 256
experts; the rank owns experts 0..31 and their weights are ``dsv3``'s experts
0..31.

Every tensor takes its own child seed from ``SeedSequence(seed).spawn``; each
expert's weights take a grandchild seed, so any single expert can be
regenerated alone and the large configurations can be drawn in parallel.
Values are drawn in float32; bf16 tensors are rounded to nearest-even and kept
as ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

# child-seed slots, in draw order
_X, _WR, _WGU, _WD, _SHARED, _BIAS, _ZIPF, _DY = range(8)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    d: int                 # d_model
    E: int                 # routed experts
    k: int                 # experts chosen per token
    f: int                 # routed expert FFN width
    dtype: str             # "f32" | "bf16": x, expert weights, activations
    score: str             # "softmax" | "sigmoid" | "sqrt_softplus"
    w_std: float           # std of every weight (router included)
    seed: int
    shared: int = 0        # shared experts applied to every token
    f_shared: int = 0
    bias: str = "zero"     # "zero" | "uniform" (U(-bias_range, bias_range))
    bias_range: float = 0.05
    bias_update: bool = False
    gamma: float = 1e-3
    zipf_s: Optional[float] = None   # logit offset 0.5*ln(rank^-s) when set
    zipf_scale: float = 0.5
    train: bool = False

    @property
    def A(self) -> int:
        """Number of (token, expert) assignments."""
        return self.T * self.k


CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=32, E=8, k=2, f=64, dtype="f32",
                      score="softmax", w_std=0.02, seed=0, bias="uniform"),
    "coarse": MoEConfig("coarse", T=4096, d=4096, E=8, k=2, f=14336, dtype="bf16",
                        score="softmax", w_std=0.02, seed=1),
    "fine": MoEConfig("fine", T=8192, d=2048, E=64, k=8, f=1024, dtype="bf16",
                      score="sigmoid", w_std=0.02, seed=2, bias_update=True,
                      zipf_s=1.2),
    "dsv3": MoEConfig("dsv3", T=4096, d=7168, E=256, k=8, f=2048, dtype="bf16",
                      score="sigmoid", w_std=0.006, seed=3, shared=1, f_shared=2048,
                      bias="uniform"),
    "train": MoEConfig("train", T=16384, d=2048, E=64, k=8, f=1024, dtype="bf16",
                       score="sqrt_softplus", w_std=0.02, seed=4, bias_update=True,
                       train=True),
}
CONFIGS["tiny_dense"] = replace(CONFIGS["tiny"], name="tiny_dense", E=1, k=1)
# the training shape under the fine workload's skewed load: the same Zipf
# logit offset (0.5 * ln(rank^-1.2) for a random rank of each expert)
CONFIGS["train_skew"] = replace(CONFIGS["train"], name="train_skew", zipf_s=1.2)


def scaled(cfg: MoEConfig, **changes) -> MoEConfig:
    """A copy of ``cfg`` with some fields replaced (used for small parity cases)."""
    return replace(cfg, **changes)


# ----------------------------------------------------------------------------
# storage helpers (bit patterns only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(ss: np.random.SeedSequence, shape, std: float, bf16: bool) -> np.ndarray:
    rng = np.random.default_rng(ss)
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    a = a.reshape(shape)
    return f32_to_bf16_bits(a) if bf16 else a


def _children(cfg: MoEConfig):
    return np.random.SeedSequence(cfg.seed).spawn(8)


def expert_weights(cfg: MoEConfig, e: int):
    """Gate/up ``[2f, d]`` and down ``[d, f]`` weights of routed expert ``e``
    (nn.Linear layout: rows are outputs, the input dimension is contiguous;
    the first f gate/up rows are the gate, the next f the up projection)."""
    kids = _children(cfg)
    bf = cfg.dtype == "bf16"
    s_gu = kids[_WGU].spawn(cfg.E)[e]
    s_d = kids[_WD].spawn(cfg.E)[e]
    return (_normal(s_gu, (2 * cfg.f, cfg.d), cfg.w_std, bf),
            _normal(s_d, (cfg.d, cfg.f), cfg.w_std, bf))


def shared_weights(cfg: MoEConfig, s: int):
    kids = _children(cfg)
    bf = cfg.dtype == "bf16"
    gu_k, d_k = kids[_SHARED].spawn(2)
    return (_normal(gu_k.spawn(cfg.shared)[s], (2 * cfg.f_shared, cfg.d), cfg.w_std, bf),
            _normal(d_k.spawn(cfg.shared)[s], (cfg.d, cfg.f_shared), cfg.w_std, bf))


EP_SHARDS = {"dsv3_ep8": ("dsv3", 8, 0)}


def ep_shard(name: str):
    """(global-batch config, first expert, end expert) of one expert-parallel
    rank: the base shape with ranks x its tokens, and the rank's contiguous
    block of E / ranks experts."""
    base, ranks, rank = EP_SHARDS[name]
    cfg = CONFIGS[base]
    per = cfg.E // ranks
    return replace(cfg, T=cfg.T * ranks), rank * per, (rank + 1) * per


def expert_weight_range(cfg: MoEConfig, e0: int, e1: int, workers: Optional[int] = None):
    """Stacked weights of routed experts e0..e1-1 (as ``make_inputs`` draws them)."""
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    wgu = np.empty((e1 - e0, 2 * cfg.f, cfg.d), dt)
    wd = np.empty((e1 - e0, cfg.d, cfg.f), dt)

    def fill(e):
        wgu[e - e0], wd[e - e0] = expert_weights(cfg, e)

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(fill, range(e0, e1)))
    return wgu, wd


def make_inputs(cfg: MoEConfig, experts: bool = True, workers: Optional[int] = None) -> dict:
    """All inputs of one layer call, as numpy arrays.

    Keys: ``x`` [T,d], ``w_router`` [E,d] f32, ``w_gate_up`` [E,2f,d], ``w_down``
    [E,d,f], ``bias`` [E] f32, ``logit_offset`` [E] f32 or None, and when set
    ``w_gate_up_shared`` [S,2fs,d], ``w_down_shared`` [S,d,fs], ``dy`` [T,d].
    bf16 tensors are uint16 bit patterns.  ``experts=False`` skips the routed
    and shared expert weights (for routing-only work on large shapes).
    """
    kids = _children(cfg)
    bf = cfg.dtype == "bf16"
    out = {
        "x": _normal(kids[_X], (cfg.T, cfg.d), 1.0, bf),
        "w_router": _normal(kids[_WR], (cfg.E, cfg.d), cfg.w_std, False),
    }
    if experts:
        dt = np.uint16 if bf else np.float32
        wgu = np.empty((cfg.E, 2 * cfg.f, cfg.d), dt)
        wd = np.empty((cfg.E, cfg.d, cfg.f), dt)

        def fill(e):
            wgu[e], wd[e] = expert_weights(cfg, e)

        with ThreadPoolExecutor(workers or _workers()) as ex:
            list(ex.map(fill, range(cfg.E)))
        out["w_gate_up"], out["w_down"] = wgu, wd
        if cfg.shared:
            sh = [shared_weights(cfg, s) for s in range(cfg.shared)]
            out["w_gate_up_shared"] = np.stack([a for a, _ in sh])
            out["w_down_shared"] = np.stack([b for _, b in sh])
    rb = np.random.default_rng(kids[_BIAS])
    if cfg.bias == "uniform":
        out["bias"] = rb.uniform(-cfg.bias_range, cfg.bias_range, cfg.E).astype(np.float32)
    else:
        out["bias"] = np.zeros(cfg.E, np.float32)
    if cfg.zipf_s is not None:
        ranks = np.random.default_rng(kids[_ZIPF]).permutation(cfg.E) + 1
        # a logit offset is a log-weight: scale * ln(rank^-s)
        out["logit_offset"] = (cfg.zipf_scale * (-cfg.zipf_s) * np.log(ranks.astype(np.float64))).astype(np.float32)
    else:
        out["logit_offset"] = None
    if cfg.train:
        out["dy"] = _normal(kids[_DY], (cfg.T, cfg.d), 1.0, True)
    return out
