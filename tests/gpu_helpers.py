"""Shared helpers of the GPU parity tests: host<->device transfer of the seeded
inputs and the comparison rules.

Comparison rules:
* expert indices, counts, offsets, row maps and permuted rows: bit-exact;
  a token whose k-th and (k+1)-th biased keys (oracle, fp64) differ by less
  than 1e-6 relative is excluded from the index comparison and counted;
* fp32 layers: max-abs and relative-L2 error <= 1e-4;
* bf16 layers: max-abs <= 2e-2 and relative-L2 <= 1e-2;
* where a floating-point value decides a bf16 rounding (a quantised code:
  H = bf16(silu(G) U) on the GPU from fp32, in the oracle from fp64), a value
  within a hair of a rounding midpoint may round either way and both results
  are correct.  rounding_ambiguous flags such values (within 2^-16 relative,
  several times the GPU's fp32 error), and a quantity summed over them gets
  the exact effect of flipping every flagged one as extra allowance
  (dg_flip_allowance for the gate gradient over H, wgrad_flip_allowance for
  the expert weight gradients over dY_perm, H and dG|dU); this is the
  rounding analogue of the near-tie rule;
* gates and logits (fp32 in every layer): max-abs <= 1e-4.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

NEAR_TIE = 1e-6
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    a = np.asarray(a)
    return oracle.bf16_from_bits(a) if a.dtype == np.uint16 else a.astype(np.float64)


def close_errors(got, ref):
    """(max-abs, relative-L2, argmax index) of got against ref."""
    got = as_f64(got)
    ref = as_f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    return mx, rel, (np.unravel_index(int(err.argmax()), err.shape) if err.size else None)


def rounding_ambiguous(v, rel=2.0 ** -16):
    """(mask, ulp): values within rel*|v| of a bf16 rounding midpoint (8
    significant bits), and the bf16 unit at each value (the size of a flip)."""
    v = np.abs(np.asarray(v, np.float64))
    m, e = np.frexp(v)                    # v = m 2^e, 0.5 <= m < 1
    scaled = m * 256.0                    # the 8-bit significand, with its fraction
    ulp = np.ldexp(1.0, e - 8)
    dist = np.abs(scaled - np.floor(scaled) - 0.5) * ulp
    return (dist <= rel * v) & (v > 0), ulp


def _flips(raw):
    """Per element: the change a flip of its bf16 rounding would make (ulp
    where the value is rounding-ambiguous, else 0)."""
    amb, ulp = rounding_ambiguous(raw)
    return np.where(amb, ulp, 0.0)


def wgrad_flip_allowance(fw, g, x):
    """Per weight-gradient element, the largest change that flipping every
    rounding-ambiguous bf16 input of its sum could cause.  dW_down[e] =
    dY_perm^T H over e's rows, with both factors bf16-rounded from fp32 (GPU)
    or fp64 (oracle) values: |flips(dY_perm)|^T |H| + |dY_perm|^T |flips(H)|.
    dW_gate_up[e] = [dG|dU]^T x, x exact: |flips(dG|dU)|^T |x|.  From the
    oracle's unrounded values."""
    offs = fw["offsets"]
    x64 = np.abs(as_f64(x))
    tok = fw["token_of"]
    ad = np.zeros(g["dw_down"].shape)
    au = np.zeros(g["dw_gate_up"].shape)
    for e in range(len(offs) - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        dyp, h = g["dy_perm"][a:b], fw["H"][a:b]
        ad[e] = _flips(g["dy_perm_raw"][a:b]).T @ np.abs(h) + np.abs(dyp).T @ _flips(fw["H_raw"][a:b])
        au[e] = _flips(g["dgu_raw"][a:b]).T @ x64[tok[a:b]]
    return ad, au


def dg_flip_allowance(fw, dy, w_down, token_of):
    """Per (token, slot): the largest change of dg = <dy[t], Y[row]> that
    flipping every rounding-ambiguous element of the row's H could cause,
    sum over those columns c of ulp(H[r,c]) * |(dy[t] W_down[e])[c]|, from the
    oracle's unrounded H."""
    offs, row_of = fw["offsets"], fw["row_of"]
    amb, ulp = rounding_ambiguous(fw["H_raw"])
    per_row = np.zeros(len(token_of))
    dy64 = as_f64(dy)
    for e in range(len(offs) - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        m = amb[a:b]
        if not m.any():
            continue
        dh = dy64[token_of[a:b]] @ as_f64(w_down[e])           # dy W_down for each row of e
        per_row[a:b] = np.sum(np.where(m, ulp[a:b] * np.abs(dh), 0.0), axis=1)
    out = np.zeros(row_of.shape)
    keep = row_of >= 0
    out[keep] = per_row[row_of[keep]]
    return out


def check_close(got, ref, kind, name):
    got = as_f64(got)
    ref = as_f64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    tol_abs, tol_rel = TOL[kind]
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    say(f"  {name}: max-abs {mx:.3e} rel-L2 {rel:.3e} (tol {tol_abs:g}/{tol_rel:g})")
    assert mx <= tol_abs and rel <= tol_rel, (name, mx, rel)
    return mx, rel


def check_route(idx, gate, logits, ref, k):
    """Compare GPU routing with the oracle's.  Returns the excluded count."""
    idx = np.asarray(idx)
    gate = np.asarray(gate, np.float64)
    excl = ref["margin"] < NEAR_TIE
    o_g = np.argsort(idx, axis=1, kind="stable")
    o_r = np.argsort(ref["idx"], axis=1, kind="stable")
    gi = np.take_along_axis(idx, o_g, 1)
    ri = np.take_along_axis(ref["idx"], o_r, 1)
    bad = np.any(gi != ri, axis=1) & ~excl
    assert not bad.any(), f"{int(bad.sum())} tokens choose different experts, first {np.nonzero(bad)[0][:5]}"
    ok = ~excl
    gg = np.take_along_axis(gate, o_g, 1)[ok]
    rg = np.take_along_axis(ref["gates"], o_r, 1)[ok]
    gerr = float(np.abs(gg - rg).max()) if gg.size else 0.0
    lerr = float(np.abs(np.asarray(logits, np.float64) - ref["logits"]).max())
    # slot order: keys descending, equal keys to the lower index (oracle keys)
    keys = np.take_along_axis(ref["keys"], idx.astype(np.int64), 1)
    for j in range(k - 1):
        a, b = keys[:, j], keys[:, j + 1]
        rel = np.abs(a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-300)
        wrong = ((a < b) | ((a == b) & (idx[:, j] > idx[:, j + 1]))) & (rel >= NEAR_TIE) & ok
        assert not wrong.any(), "slot order differs"
    say(f"  route: excluded near-ties {int(excl.sum())}, gate max-abs {gerr:.2e}, logit max-abs {lerr:.2e}")
    assert gerr <= 1e-4 and lerr <= 1e-4, (gerr, lerr)
    return int(excl.sum())


def check_permute(idx, E, counts, offsets, row_of, token_of, x_perm, x, capacity=None):
    """Stage-isolated: the oracle permute fed the GPU's own choice."""
    c, o, r, t = oracle.permute(np.asarray(idx, np.int64), E, capacity)
    assert np.array_equal(np.asarray(counts), c), "counts"
    assert np.array_equal(np.asarray(offsets), o), "offsets"
    assert np.array_equal(np.asarray(row_of), r), "row_of"
    assert np.array_equal(np.asarray(token_of), t), "token_of"
    assert np.array_equal(np.asarray(x_perm), np.asarray(x)[t]), "x_perm"
