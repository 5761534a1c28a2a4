"""The MoE layer's forward in plain Python loops, for small cases (test
infrastructure only, like the rest of ``oracle``).

It shares no code with ``oracle.moe``: it takes nested lists of Python floats
(float64), uses only ``math``, and goes a different way to the same result,
so each one checks the other.  Per token: the router's logits and scores,
the k largest selection keys picked one at a time (ties to the lower expert
index), the gates, then each chosen expert applied to the token itself (no
permutation) and the gated sum.

Pages (titles): the "专家组合 (MoE)" lesson, AI Engineering from Scratch --
Concept (a router picks k of E experts per token and the layer adds the
gate-weighted expert outputs), Build it step 1 (bias only in the selection
key; gates from the raw scores of the chosen experts; ties to the lower
index), Shared experts (every token also passes through them) and Key terms
(an expert is a SwiGLU FFN); the AREX article on The Ultimate MoE Training
Handbook, router-precision paragraph (sigmoid and sqrt(softplus) scores).
"""
from __future__ import annotations

import math


def score(l: float, fn: str) -> float:
    """Router score of one logit: the logit itself (softmax routing takes the
    softmax over the chosen experts later), the logistic sigmoid, or
    sqrt(ln(1 + e^l))."""
    if fn == "softmax":
        return l
    if fn == "sigmoid":
        return 1.0 / (1.0 + math.exp(-l)) if l >= 0 else math.exp(l) / (1.0 + math.exp(l))
    if fn == "sqrt_softplus":
        return math.sqrt(max(l, 0.0) + math.log1p(math.exp(-abs(l))))
    raise ValueError(fn)


def bf16(v: float) -> float:
    """v rounded to 8 significant bits, ties to even (bf16 storage)."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)            # v = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0) / 256.0, e)   # round(): half to even


def dot(a, b) -> float:
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def route_token(xt, w_router, k: int, fn: str, bias=None, offset=None):
    """(chosen experts in slot order, their gates) for one token."""
    E = len(w_router)
    logits = [dot(xt, w_router[e]) + (offset[e] if offset is not None else 0.0) for e in range(E)]
    scores = [score(l, fn) for l in logits]
    keys = [scores[e] + (bias[e] if bias is not None else 0.0) for e in range(E)]
    chosen = []
    for _ in range(k):
        best = -1
        for e in range(E):          # ascending: a later expert must beat, not tie
            if e in chosen:
                continue
            if best < 0 or keys[e] > keys[best]:
                best = e
        chosen.append(best)
    if fn == "softmax":
        top = max(logits[e] for e in chosen)
        w = [math.exp(logits[e] - top) for e in chosen]
    else:
        w = [scores[e] for e in chosen]
    tot = sum(w)
    return chosen, [v / tot for v in w]


def swiglu_expert(xt, w_gate_up, w_down, bf16_points: bool):
    """One SwiGLU expert on one token: the gate and up rows are the first and
    second f rows of w_gate_up [2f][d]; H = silu(gate) * up (bf16-stored when
    bf16_points); y = w_down [d][f] applied to H."""
    f = len(w_down[0])
    h = []
    for j in range(f):
        g = dot(xt, w_gate_up[j])
        u = dot(xt, w_gate_up[f + j])
        v = g / (1.0 + math.exp(-g)) * u if g >= -700.0 else 0.0
        h.append(bf16(v) if bf16_points else v)
    return [dot(h, w_down[c]) for c in range(len(w_down))]


def forward(x, w_router, w_gate_up, w_down, k: int, score_fn: str, bf16_points: bool,
            sel_bias=None, logit_offset=None, w_gate_up_shared=None, w_down_shared=None) -> dict:
    """out[t] = sum over the shared experts of their output
             + sum over the chosen experts e_j of gate_j * expert_{e_j}(x[t])."""
    idx, gates, out = [], [], []
    for xt in x:
        chosen, g = route_token(xt, w_router, k, score_fn, sel_bias, logit_offset)
        o = [0.0] * len(xt)
        for s in range(len(w_gate_up_shared or [])):
            ys = swiglu_expert(xt, w_gate_up_shared[s], w_down_shared[s], bf16_points)
            o = [o[c] + ys[c] for c in range(len(o))]
        for j, e in enumerate(chosen):
            ye = swiglu_expert(xt, w_gate_up[e], w_down[e], bf16_points)
            o = [o[c] + g[j] * ye[c] for c in range(len(o))]
        idx.append(chosen)
        gates.append(g)
        out.append(o)
    return {"idx": idx, "gates": gates, "out": out}
