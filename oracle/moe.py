"""Plain fp64 reference of the token-choice MoE layer (test infrastructure only).

Notation: T tokens, d model width, E routed experts, k experts per token,
f expert FFN width, A = T*k (token, expert) assignments.

Where the pages leave a step open, the reading taken is stated at the function.
Everything is computed in float64.  For layers whose storage type is bf16 the
oracle rounds to bf16 exactly where such a layer stores a bf16 tensor
(``bf16_points=True``): the saved gate/up pre-activations G and U, the SwiGLU
output H, the gate-scaled output gradient dY_perm (the input of W_down's
weight gradient; the data gradient scales dY W_down by the gate instead),
the SwiGLU input gradients dG, dU, and each expert row's input gradient
dX_perm (its k rows per token are summed in high precision).  Expert outputs, the combined output and every gradient that
leaves the layer stay in high precision.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

SCORE_FNS = ("softmax", "sigmoid", "sqrt_softplus")


# ----------------------------------------------------------------------------
# bf16 storage (the oracle's own conversion; checked against torch in the tests)

def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """Value of uint16 bf16 bit patterns, as float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits,
    ties to even), returned as float64.  Finite normal range only."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)   # np.rint rounds half to even


def _f64(a: np.ndarray) -> np.ndarray:
    """Inputs arrive as float32/float64 arrays or as uint16 bf16 bit patterns."""
    a = np.asarray(a)
    return bf16_from_bits(a) if a.dtype == np.uint16 else a.astype(np.float64)


# ----------------------------------------------------------------------------
# routing — lesson "专家组合 (MoE)", Concept and Build it step 1; router score
# functions and fp32 rule from the AREX article's router-precision paragraph.

def score(logits: np.ndarray, fn: str) -> np.ndarray:
    """Router score of each logit.

    softmax: the raw logit itself (the softmax is taken later, over the chosen
    experts only, as the lesson's router does); sigmoid: 1/(1+e^-l);
    sqrt_softplus: sqrt(ln(1+e^l)), with ln(1+e^l) = max(l,0) + ln(1+e^-|l|)
    (the two pages only name the last two functions; these are their standard
    definitions)."""
    l = np.asarray(logits, dtype=np.float64)
    if fn == "softmax":
        return l.copy()
    if fn == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    if fn == "sqrt_softplus":
        return np.sqrt(np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l))))
    raise ValueError(fn)


def route(x, w_router, k: int, score_fn: str, sel_bias=None, logit_offset=None) -> dict:
    """Router, top-k and gates for every token.

    * logits l = x . W_r^T (+ a per-expert logit offset, used by synthetic
      skewed workloads; it is part of the raw logit);
    * selection key = score + bias: the loss-free bias moves which experts are
      chosen but never enters the gate (lesson, Load balancing, and the remark
      after Build it step 1);
    * the k largest keys are chosen by a stable sort on -key, so equal keys go
      to the lower expert index; slot order is the sort order;
    * gates: softmax over the chosen experts' raw logits (lesson, step 1) for
      ``softmax``; otherwise each chosen score divided by the sum of the chosen
      scores.

    Returns idx [T,k] int64, gates [T,k], logits [T,E], scores [T,E],
    keys [T,E], margin [T] = |key_(k) - key_(k+1)| / max(|key_(k)|, |key_(k+1)|)
    (0 when both are 0, +inf when k == E).
    """
    x = _f64(x)
    w = _f64(w_router)
    T = x.shape[0]
    E = w.shape[0]
    assert 1 <= k <= E
    logits = x @ w.T
    if logit_offset is not None:
        logits = logits + _f64(logit_offset)[None, :]
    s = score(logits, score_fn)
    b = np.zeros(E) if sel_bias is None else _f64(sel_bias)
    keys = s + b[None, :]
    idx = np.empty((T, k), np.int64)
    gates = np.empty((T, k))
    margin = np.full(T, np.inf)
    for t in range(T):
        order = np.argsort(-keys[t], kind="stable")
        chosen = order[:k]
        idx[t] = chosen
        if k < E:
            a, c = keys[t, order[k - 1]], keys[t, order[k]]
            den = max(abs(a), abs(c))
            margin[t] = abs(a - c) / den if den > 0 else 0.0
        if score_fn == "softmax":
            raw = logits[t, chosen]
            ex = np.exp(raw - raw.max())
            gates[t] = ex / ex.sum()
        else:
            sc = s[t, chosen]
            gates[t] = sc / sc.sum()
    return {"idx": idx, "gates": gates, "logits": logits, "scores": s,
            "keys": keys, "margin": margin}


# ----------------------------------------------------------------------------
# hash router — lesson, Exercises item 2: replace the learned router by a
# deterministic hash of the token, nothing learned.  The hash is SplitMix64
# (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
# OOPSLA 2014): the generator adds 0x9E3779B97F4A7C15 to its state and mixes.

_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def splitmix_key(ids, experts, salt: int = 0) -> np.ndarray:
    """Output number salt+1 of SplitMix64 started at state id*2^32 + e."""
    ids = np.asarray(ids, np.int64).astype(np.uint32).astype(np.uint64)
    experts = np.asarray(experts, np.uint64)
    state = (ids << np.uint64(32)) | experts
    with np.errstate(over="ignore"):
        z = state + np.uint64(salt + 1) * _GAMMA                  # uint64 arithmetic wraps mod 2^64
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def hash_route(token_ids, E: int, k: int, salt: int = 0) -> dict:
    """Each token takes the k experts with the smallest keys splitmix_key(id, e),
    ascending (lower expert first on a tie), with equal gates 1/k."""
    ids = np.asarray(token_ids, np.int64)
    T = len(ids)
    keys = splitmix_key(ids[:, None], np.arange(E)[None, :], salt)
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        idx[t] = np.argsort(keys[t], kind="stable")[:k]
    return {"idx": idx, "gates": np.full((T, k), 1.0 / k)}


# ----------------------------------------------------------------------------
# permute — grouping the (token, expert) pairs by expert ahead of the expert
# GEMMs (the "permute" the AREX article's permute-fusion paragraph refers to).

def permute(idx: np.ndarray, E: int, capacity=None):
    """Stable counting sort of the T*k assignments by expert.

    counts[e] = number of assignments to e; offsets = exclusive prefix sum
    (length E+1).  Experts are walked in ascending order and, inside an expert,
    tokens in ascending order (the pages do not fix this order; ascending token
    order makes the permutation unique).  Assignment (t, j) takes row
    row_of[t, j]; token_of[row] = t.

    Expert capacity (lesson, Load balancing item 2: an expert processes at
    most a fixed number of tokens and the overflow skips the layer): with
    ``capacity`` c, expert e keeps its first min(counts[e], c) assignments in
    token order and drops the others.  ``offsets`` then sums the kept counts;
    kept rows fill 0 .. offsets[E]-1 and the dropped rows follow, grouped by
    expert the same way.  A dropped assignment's row r is recorded as ~r
    (negative); ``counts`` still counts every assignment."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(idx == e))
    if capacity is None or capacity < 0:
        kept = counts.copy()
    else:
        kept = np.minimum(counts, capacity)
    dropped = counts - kept
    offsets = np.zeros(E + 1, np.int64)
    dstart = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
        dstart[e + 1] = dstart[e] + dropped[e]
    row_of = np.full((T, k), np.iinfo(np.int32).min, np.int64)
    token_of = np.full(T * k, -1, np.int64)
    for e in range(E):
        ts, js = np.nonzero(idx == e)      # row-major: tokens ascending
        n = int(kept[e])
        rows = offsets[e] + np.arange(n)
        row_of[ts[:n], js[:n]] = rows
        token_of[rows] = ts[:n]
        drows = offsets[E] + dstart[e] + np.arange(len(ts) - n)
        row_of[ts[n:], js[n:]] = ~drows
        token_of[drows] = ts[n:]
    return counts, offsets, row_of, token_of


# ----------------------------------------------------------------------------
# experts — each expert is an independent SwiGLU FFN (lesson, Concept; Key
# terms "Expert").  Weight layout: w_gate_up [2f, d] (gate rows, then up rows),
# w_down [d, f].

def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xr, w_gate_up, w_down, bf16_points: bool) -> dict:
    """SwiGLU expert on rows xr [n, d]: G = xr Wg^T, U = xr Wu^T,
    H = silu(G) * U (computed from the unrounded G and U), Y = H Wd^T.
    Returns G, U (saved form: bf16-rounded when bf16_points), H, Y, and
    H_raw (H before its bf16 rounding)."""
    xr = _f64(xr)
    wgu = _f64(w_gate_up)
    wd = _f64(w_down)
    f = wd.shape[1]
    G = xr @ wgu[:f].T
    U = xr @ wgu[f:].T
    H_raw = _silu(G) * U
    if bf16_points:
        H = bf16_round(H_raw)
        Gs, Us = bf16_round(G), bf16_round(U)
    else:
        H, Gs, Us = H_raw, G, U
    Y = H @ wd.T
    return {"G": Gs, "U": Us, "H": H, "Y": Y, "H_raw": H_raw}


def grouped_ffn(x_perm, offsets, w_gate_up, w_down, bf16_points: bool) -> dict:
    """Expert e applied to rows offsets[e]:offsets[e+1] of x_perm."""
    x_perm = _f64(x_perm)
    G_ = len(offsets) - 1
    A = x_perm.shape[0]
    f = np.asarray(w_down).shape[2]
    d = np.asarray(w_down).shape[1]
    out = {"G": np.zeros((A, f)), "U": np.zeros((A, f)), "H": np.zeros((A, f)), "H_raw": np.zeros((A, f)),
           "Y": np.zeros((A, d))}
    for e in range(G_):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        r = expert_ffn(x_perm[a:b], w_gate_up[e], w_down[e], bf16_points)
        for key in out:
            out[key][a:b] = r[key]
    return out


# ----------------------------------------------------------------------------
# combine — out = sum over the chosen experts of gate * expert output, plus the
# shared experts every token passes through (lesson, Concept and Shared
# experts).  The residual add sits outside the layer.

def combine(y_perm, row_of, gates, shared_y=None):
    """out[t] = shared_y[t] + sum over the kept slots j of gate[t,j] * y[row_of[t,j]];
    a dropped slot (row_of < 0) adds nothing: the token skips the layer there."""
    y_perm = np.asarray(y_perm, np.float64)
    gates = np.asarray(gates, np.float64)
    T, k = row_of.shape
    out = np.zeros((T, y_perm.shape[1])) if shared_y is None else np.array(shared_y, np.float64)
    for j in range(k):
        keep = row_of[:, j] >= 0
        out[keep] += gates[keep, j:j + 1] * y_perm[row_of[keep, j]]
    return out


# ----------------------------------------------------------------------------
# loss-free balancing bias controller (lesson, Load balancing item 3 and Build
# it step 2)

def bias_update(bias, counts, T: int, k: int, gamma: float) -> np.ndarray:
    """After a step, an expert used more than the uniform target T*k/E moves its
    bias down by gamma, one used less moves it up, one exactly on target keeps
    it.  The target comparison is done in integers (E*count vs T*k); the update
    is one float32 add, as the bias is stored in float32."""
    b = np.array(bias, dtype=np.float32)
    E = b.shape[0]
    g = np.float32(gamma)
    for e in range(E):
        load = E * int(counts[e])
        if load > T * k:
            b[e] = np.float32(b[e] - g)
        elif load < T * k:
            b[e] = np.float32(b[e] + g)
    return b


# ----------------------------------------------------------------------------
# whole forward

def forward(x, w_router, w_gate_up, w_down, k: int, score_fn: str, bf16_points: bool,
            sel_bias=None, logit_offset=None, w_gate_up_shared=None, w_down_shared=None,
            idx=None, capacity=None) -> dict:
    """Route, permute, run the experts, add the shared experts, combine.

    ``idx`` forces the expert choice (stage-isolated checks feed the GPU's own
    choice); gates are then recomputed for that choice.  ``capacity`` caps the
    rows of each expert (see ``permute``)."""
    if score_fn == "uniform":           # hash routing: the choice is given, gates are 1/k
        idx = np.asarray(idx, np.int64)
        E = np.asarray(w_gate_up).shape[0]
        T = idx.shape[0]
        r = {"idx": idx, "gates": np.full((T, k), 1.0 / k), "logits": None, "scores": None,
             "margin": np.full(T, np.inf)}
    else:
        E = np.asarray(w_router).shape[0]
        r = route(x, w_router, k, score_fn, sel_bias, logit_offset)
    if idx is not None and score_fn != "uniform":
        idx = np.asarray(idx, np.int64)
        r["idx"] = idx
        r["gates"] = _gates_for(r, idx, score_fn)
    counts, offsets, row_of, token_of = permute(r["idx"], E, capacity)
    x64 = _f64(x)
    x_perm = x64[token_of]
    ex = grouped_ffn(x_perm, offsets, w_gate_up, w_down, bf16_points)
    shared_y = None
    sh = []
    if w_gate_up_shared is not None:
        shared_y = np.zeros_like(x64)
        for s in range(len(w_gate_up_shared)):
            o = expert_ffn(x64, w_gate_up_shared[s], w_down_shared[s], bf16_points)
            sh.append(o)
            shared_y += o["Y"]
    out = combine(ex["Y"], row_of, r["gates"], shared_y)
    res = dict(r)
    res.update(counts=counts, offsets=offsets, row_of=row_of, token_of=token_of,
               x_perm=x_perm, G=ex["G"], U=ex["U"], H=ex["H"], H_raw=ex["H_raw"], y_perm=ex["Y"],
               shared=sh, shared_y=shared_y, out=out)
    return res


def _gates_for(r: dict, idx: np.ndarray, score_fn: str) -> np.ndarray:
    """Gates of a given choice (routing replay, lesson Exercises item 3: the
    experts that fired are recorded and the same routing is forced later).
    A replayed choice is one the router made, so every id lies in [0, E) and a
    token holds each expert at most once; anything else is not a choice and
    is rejected."""
    T, k = idx.shape
    E = r["logits"].shape[1]
    _check_choice(idx, E)
    g = np.zeros((T, k))
    for t in range(T):
        if score_fn == "softmax":
            raw = r["logits"][t, idx[t]]
            ex = np.exp(raw - raw.max())
            g[t] = ex / ex.sum()
        else:
            sc = r["scores"][t, idx[t]]
            g[t] = sc / sc.sum()
    return g


def _check_choice(idx: np.ndarray, E: int) -> None:
    if np.any((idx < 0) | (idx >= E)):
        raise ValueError("an expert id outside [0, E) is not a routing choice")
    s = np.sort(idx, axis=1)
    if s.shape[1] > 1 and np.any(s[:, 1:] == s[:, :-1]):
        raise ValueError("a token holds the same expert twice")


# ----------------------------------------------------------------------------
# backward (chain rule through the forward above; the bias, the logit offset and
# the discrete top-k choice get no gradient — lesson, Key terms: the loss-free
# bias adds no gradient signal)

def gate_backward(dg, gates, logits_chosen, scores_chosen, score_fn: str):
    """d loss / d logit of each chosen expert, given d loss / d gate.

    softmax over the chosen: dl_j = g_j (dg_j - D), D = sum_i g_i dg_i.
    normalised scores g_j = s_j / S: ds_j = (dg_j - D) / S, then
    dl_j = ds_j * s'(l_j) with s' = s(1-s) for the sigmoid and
    sigmoid(l) / (2 s) for sqrt(softplus)."""
    dg = np.asarray(dg, np.float64)
    g = np.asarray(gates, np.float64)
    D = np.sum(g * dg, axis=1, keepdims=True)
    if score_fn == "softmax":
        return g * (dg - D)
    s = np.asarray(scores_chosen, np.float64)
    S = np.sum(s, axis=1, keepdims=True)
    ds = (dg - D) / S
    l = np.asarray(logits_chosen, np.float64)
    if score_fn == "sigmoid":
        return ds * s * (1.0 - s)
    if score_fn == "sqrt_softplus":
        return ds * (1.0 / (1.0 + np.exp(-l))) / (2.0 * s)
    raise ValueError(score_fn)


def router_backward(dl, idx, x, w_router):
    """logits = x W_r^T: dW_r = dL^T x and dx = dL W_r, with dL the [T,E]
    logit gradient that is dl at the chosen experts and zero elsewhere."""
    x = _f64(x)
    w = _f64(w_router)
    T, k = idx.shape
    E = w.shape[0]
    dL = np.zeros((T, E))
    for j in range(k):
        dL[np.arange(T), idx[:, j]] += dl[:, j]
    return dL.T @ x, dL @ w


def expert_backward_rows(dy_rows, xr, G, U, H, w_gate_up, w_down, bf16_points: bool, dy_wgrad=None) -> dict:
    """Backward of one SwiGLU expert over rows xr, given d loss / d Y rows.

    dH = dY Wd; dG = dH * U * silu'(G); dU = dH * silu(G) (G, U in their saved
    form); dWd = dY^T H; dWg = dG^T xr; dWu = dU^T xr; dX = dG Wg + dU Wu.
    silu'(z) = sigma(z) (1 + z (1 - sigma(z))).
    dy_wgrad: the form of dY that the weight gradient dWd uses when it differs
    from the one the data gradient uses (a bf16-stored copy); default dy_rows."""
    xr = _f64(xr)
    wgu = _f64(w_gate_up)
    wd = _f64(w_down)
    f = wd.shape[1]
    dy = np.asarray(dy_rows, np.float64)
    dyw = dy if dy_wgrad is None else np.asarray(dy_wgrad, np.float64)
    dH = dy @ wd
    sg = 1.0 / (1.0 + np.exp(-G))
    dG_raw = dH * U * sg * (1.0 + G * (1.0 - sg))
    dU_raw = dH * (G * sg)
    if bf16_points:
        dG, dU = bf16_round(dG_raw), bf16_round(dU_raw)
    else:
        dG, dU = dG_raw, dU_raw
    dX = dG @ wgu[:f] + dU @ wgu[f:]
    dWgu = np.concatenate([dG.T @ xr, dU.T @ xr], axis=0)
    dWd = dyw.T @ H
    return {"dH": dH, "dG": dG, "dU": dU, "dX": dX, "dW_gate_up": dWgu, "dW_down": dWd,
            "dGU_raw": np.concatenate([dG_raw, dU_raw], axis=1)}


def backward(fwd: dict, dy, x, w_router, w_gate_up, w_down, score_fn: str,
             bf16_points: bool, w_gate_up_shared=None, w_down_shared=None, aux_alpha: float = 0.0) -> dict:
    """Gradients of sum(out * dy) with respect to x and every weight.

    combine:   dg[t,j] = <dy[t], Y[row_of[t,j]]>, dY_perm[row_of[t,j]] = g[t,j] dy[t]
    gates:     dl via gate_backward; router: dW_r, dx_r via router_backward
    experts:   expert_backward_rows per expert segment
    unpermute: dx[t] = sum_j dX_perm[row_of[t,j]] + dx_r[t] (+ shared experts' dX)
    Dropped slots (capacity) contribute to neither sum over experts; their
    logits still get dl through the gate normalisation.
    aux_alpha > 0 adds the auxiliary loss (``aux_loss``): its gradient reaches
    every logit, so the router gradients use the dense [T, E] logit gradient
    (returned as "dl_dense").
    """
    dy = _f64(dy)
    idx, gates, row_of = fwd["idx"], fwd["gates"], fwd["row_of"]
    T, k = idx.shape
    E = len(fwd["counts"])
    A = T * k
    d = dy.shape[1]
    y = fwd["y_perm"]
    dg = np.zeros((T, k))
    dy_perm = np.zeros((A, d))
    for j in range(k):
        keep = row_of[:, j] >= 0          # a dropped slot has no expert output: dg = 0
        dg[keep, j] = np.sum(dy[keep] * y[row_of[keep, j]], axis=1)
        dy_perm[row_of[keep, j]] = gates[keep, j:j + 1] * dy[keep]
    # bf16 layers store g*dY in bf16 for the weight gradient of W_down only;
    # the data gradient scales dY W_down by g in high precision
    dy_perm_w = bf16_round(dy_perm) if bf16_points else dy_perm
    if score_fn == "uniform":           # constant gates: no logit and no router gradient
        dl = np.zeros((T, k))
        dW_r, dx = np.zeros((E, d)), np.zeros((T, d))
    else:
        _check_choice(idx, E)
        tt = np.arange(T)[:, None]
        lc = fwd["logits"][tt, idx]
        sc = fwd["scores"][tt, idx]
        dl = gate_backward(dg, gates, lc, sc, score_fn)
        if aux_alpha:
            dL = np.zeros((T, E))
            np.add.at(dL, (np.arange(T)[:, None].repeat(k, 1), idx), dl)
            dL += aux_grad_logits(fwd["logits"], fwd["counts"], k, score_fn, aux_alpha)
            dW_r, dx = dL.T @ _f64(x), dL @ np.asarray(w_router, np.float64)
        else:
            dW_r, dx = router_backward(dl, idx, x, w_router)
    f = np.asarray(w_down).shape[2]
    dW_gu = np.zeros((E, 2 * f, d))
    dW_d = np.zeros((E, d, f))
    dX_perm = np.zeros((A, d))
    dGU = np.zeros((A, 2 * f))
    dGU_raw = np.zeros((A, 2 * f))
    offs = fwd["offsets"]
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a == b:
            continue
        r = expert_backward_rows(dy_perm[a:b], fwd["x_perm"][a:b], fwd["G"][a:b], fwd["U"][a:b],
                                 fwd["H"][a:b], w_gate_up[e], w_down[e], bf16_points, dy_wgrad=dy_perm_w[a:b])
        dW_gu[e], dW_d[e] = r["dW_gate_up"], r["dW_down"]
        dX_perm[a:b] = r["dX"]
        dGU[a:b, :f], dGU[a:b, f:] = r["dG"], r["dU"]
        dGU_raw[a:b] = r["dGU_raw"]
    # bf16 layers store each expert row's input gradient in bf16 and sum the
    # k rows of a token in high precision
    dX_rows = bf16_round(dX_perm) if bf16_points else dX_perm
    for j in range(k):
        keep = row_of[:, j] >= 0
        dx[keep] += dX_rows[row_of[keep, j]]
    # *_raw: the values before their bf16 rounding (bf16 layers)
    out = {"dx": dx, "dw_router": dW_r, "dw_gate_up": dW_gu, "dw_down": dW_d,
           "dg": dg, "dl": dl, "dy_perm": dy_perm_w, "dy_perm_raw": dy_perm, "dx_perm": dX_perm, "dgu": dGU,
           "dgu_raw": dGU_raw}
    if aux_alpha and score_fn != "uniform":
        out["dl_dense"] = dL
    if w_gate_up_shared is not None:
        x64 = _f64(x)
        out["dw_gate_up_shared"], out["dw_down_shared"] = [], []
        for s, o in enumerate(fwd["shared"]):
            r = expert_backward_rows(dy, x64, o["G"], o["U"], o["H"], w_gate_up_shared[s],
                                     w_down_shared[s], bf16_points)
            out["dx"] = out["dx"] + r["dX"]
            out["dw_gate_up_shared"].append(r["dW_gate_up"])
            out["dw_down_shared"].append(r["dW_down"])
    return out


# ----------------------------------------------------------------------------
# auxiliary load-balancing loss — lesson, Load balancing item 1 (a penalty on
# uneven expert usage, with a weight and its own gradient) and Key terms
# (auxiliary loss).  PARITY UNPINNED: the pages give no formula.  The reading
# taken is the Switch/GShard form
#     L_aux = alpha * E / (T*k) * sum_e counts[e] * P[e],
#     P[e]  = mean over tokens of p[t, e],
# with p the router probabilities over ALL E experts (softmax of the logits
# for softmax scoring; each score over the sum of all E scores otherwise) and
# counts the top-k assignments (not differentiated).  Balanced counts and
# uniform p give L_aux = alpha.

def aux_probs(logits, score_fn: str) -> np.ndarray:
    l = np.asarray(logits, np.float64)
    if score_fn == "softmax":
        ex = np.exp(l - l.max(axis=1, keepdims=True))
        return ex / ex.sum(axis=1, keepdims=True)
    s = score(l, score_fn)
    return s / s.sum(axis=1, keepdims=True)


def aux_loss(logits, counts, k: int, score_fn: str, alpha: float) -> float:
    p = aux_probs(logits, score_fn)
    T, E = p.shape
    return float(alpha * E / (T * k) * np.sum(np.asarray(counts, np.float64) * p.mean(axis=0)))


def aux_grad_logits(logits, counts, k: int, score_fn: str, alpha: float) -> np.ndarray:
    """d L_aux / d logits [T, E] (counts held fixed).  With c_e = dL/dp[t,e]
    = alpha * E / (T*k) * counts[e] / T: softmax: p_i (c_i - sum_e p_e c_e);
    normalised scores p = s / S: (c_i - sum_e p_e c_e) / S * s'(l_i)."""
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    c = alpha * E / (T * k) * np.asarray(counts, np.float64) / T
    p = aux_probs(l, score_fn)
    pc = np.sum(p * c, axis=1, keepdims=True)
    if score_fn == "softmax":
        return p * (c - pc)
    s = score(l, score_fn)
    ds = (c - pc) / s.sum(axis=1, keepdims=True)
    if score_fn == "sigmoid":
        return ds * s * (1.0 - s)
    return ds * (1.0 / (1.0 + np.exp(-l))) / (2.0 * s)


# ----------------------------------------------------------------------------
# parameter arithmetic (lesson, Fine-grained experts and Cost profile; AREX
# article, the 64-expert top-8 teaching model)

def moe_ffn_params(d: int, f: int, E: int, k: int, shared: int = 0, f_shared: int = 0):
    """(stored, active-per-token) parameters of one SwiGLU MoE layer:
    E experts of 3*d*f each, a d x E router, shared experts always active."""
    per = 3 * d * f
    sh = shared * 3 * d * f_shared
    return E * per + d * E + sh, k * per + d * E + sh


def dense_ffn_params(d: int, F: int) -> int:
    """A dense SwiGLU FFN of width F (gate, up and down projections)."""
    return 3 * d * F
