"""A token-choice MoE layer driven through the C ABI.

``MoELayer`` owns the device weights and preallocated buffers and chains the
library calls of one forward (route -> permute -> routed experts -> shared
experts -> combine -> bias update) and, for training, the backward.  It does
no arithmetic of its own: every step is a call into libmoe.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from math import ceil
from typing import Optional

import torch

from . import _lib as L


@dataclass
class Shape:
    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: torch.dtype = torch.bfloat16
    score: str = "softmax"
    shared: int = 0
    f_shared: int = 0
    bias_update: bool = False
    gamma: float = 1e-3
    train: bool = False
    capacity: Optional[int] = None   # rows per expert (token dropping); None: no cap
    router: str = "learned"          # "learned" (scores, top-k) or "hash" (token ids, gates 1/k)
    salt: int = 0                    # hash router: per-layer salt
    aux_alpha: float = 0.0           # weight of the auxiliary load-balancing loss (0: off)
    fuse_permute: bool = True        # the up-projection and W_gate_up's weight gradient gather x rows: no X_perm copy
    packed_weights: bool = False     # forward-only: expert weights packed once in tile order (moe_pack_expert_weights)


def expert_capacity(factor: float, T: int, k: int, E: int) -> int:
    """Rows per expert for a capacity factor C: ceil(C * T * k / E), evaluated
    exactly on the given float C (lesson, Load balancing item 2: C x N / E
    tokens per expert, counted here in assignments for top-k)."""
    return int(ceil(Fraction(factor) * T * k / E))


class CallTimer:
    """HIP events around library calls, on the stream the calls go to."""

    def __init__(self):
        self.pairs = {}

    def span(self, name, stream=None):
        timer = self

        class _Span:
            def __enter__(self_):
                self_.a = torch.cuda.Event(enable_timing=True)
                self_.b = torch.cuda.Event(enable_timing=True)
                self_.a.record(stream)

            def __exit__(self_, *exc):
                self_.b.record(stream)
                timer.pairs.setdefault(name, []).append((self_.a, self_.b))
        return _Span()

    def mean_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in p) / len(p) if p else float("nan")

    def reset(self):
        self.pairs = {}


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def _span(timer, name, stream):
    return timer.span(name, stream) if timer is not None else _Null()


class MoELayer:
    def __init__(self, shape: Shape, w_router, w_gate_up, w_down, sel_bias=None, logit_offset=None,
                 w_gate_up_shared=None, w_down_shared=None, device="cuda"):
        s = shape
        self.s = s
        dev = torch.device(device)
        self.dev = dev
        self.w_router = w_router
        self.w_gate_up = w_gate_up
        self.w_down = w_down
        self.sel_bias = sel_bias
        self.logit_offset = logit_offset
        self.w_gate_up_shared = w_gate_up_shared
        self.w_down_shared = w_down_shared
        T, d, E, k, f, A = s.T, s.d, s.E, s.k, s.f, s.T * s.k
        dt = s.dtype
        z = lambda *shp, dtype=torch.float32: torch.empty(shp, dtype=dtype, device=dev)
        self.idx = z(T, k, dtype=torch.int32)
        self.gate = z(T, k)
        self.logits = z(T, E)
        self.counts = z(E, dtype=torch.int32)
        self.offsets = z(E + 1, dtype=torch.int32)
        self.row_of = z(T, k, dtype=torch.int32)
        self.token_of = z(A, dtype=torch.int32)
        # the up-projection, and in training the weight gradient of W_gate_up,
        # read x through token_of (the permute fused into the expert GEMMs):
        # then no X_perm is written
        self.gather = s.fuse_permute
        # a serving layer whose weights do not change packs them once: each
        # GEMM slab is then one contiguous read (the backward reads the
        # weights unpacked, so a training layer keeps them as given)
        self.packed = self.packed_sh = None
        if s.packed_weights:
            if s.train:
                raise ValueError("packed expert weights are for forward-only layers")
            self.packed = L.moe_pack_expert_weights(w_gate_up, w_down)
            if s.shared and s.f_shared % 128 == 0:
                self.packed_sh = L.moe_pack_expert_weights(w_gate_up_shared, w_down_shared)
        self.x_perm = None if self.gather else z(A, d, dtype=dt)
        self.gu = z(A, 2 * f, dtype=dt) if s.train else None
        self.h = z(A, f, dtype=dt)
        self.y_perm = z(A, d)
        self.out = z(T, d)
        self.ws_perm = z(max(1, L.workspace_size(L.MOE_CALL_PERMUTE, T, k, E, d, f)), dtype=torch.uint8)
        self.ws_ffn = z(max(1, L.workspace_size(L.MOE_CALL_GROUPED_FFN, A, 1, E, d, f)), dtype=torch.uint8)
        if s.shared:
            # S shared SwiGLU experts of width fs sum to one expert of width
            # S*fs (gate/up rows and down columns concatenated): pass that one.
            if s.shared != 1:
                raise ValueError("pass S shared experts as one shared expert of width S*f_shared")
            fs = s.f_shared
            self.sh_offsets = torch.tensor([0, T], dtype=torch.int32, device=dev)
            self.sh_h = z(T, fs, dtype=dt)
            self.sh_y = z(T, d)
            self.ws_sh = z(max(1, L.workspace_size(L.MOE_CALL_GROUPED_FFN, T, 1, 1, d, fs)), dtype=torch.uint8)
            self.sh_gu = z(T, 2 * fs, dtype=dt) if s.train else None
            if s.train:
                self.dw_gate_up_shared = z(2 * fs, d)
                self.dw_down_shared = z(d, fs)
                self.ws_bwd_sh = z(max(1, L.workspace_size(L.MOE_CALL_BACKWARD_SHARED, T, 1, 1, d, fs)),
                                   dtype=torch.uint8)
        if s.train:
            self.dx = z(T, d)
            self.dw_router = z(E, d)
            self.dw_gate_up = z(E, 2 * f, d)
            self.dw_down = z(E, d, f)
            self.dgate = z(T, k)
            self.dlogit = z(T, k)
            self.ws_bwd = z(max(1, L.workspace_size(L.MOE_CALL_BACKWARD, T, k, E, d, f)), dtype=torch.uint8)
        if s.aux_alpha:
            self.aux_loss = z(1)
            self.aux_p = z(E)
            self.ws_aux = z(max(1, L.workspace_size(L.MOE_CALL_AUX_LOSS, T, k, E, d, f)), dtype=torch.uint8)

    def forward(self, x, stream=None, timer=None, token_ids=None, replay_idx=None, ffn_events=None):
        """One forward.  ``replay_idx`` [T, k] int32 forces the expert choice
        (routing replay); the hash router needs ``token_ids`` [T] int32.
        ``ffn_events``: None, or 1 + len(_lib.FFN_STAGES) torch.cuda.Event
        objects: the first is recorded before the routed experts' grouped FFN
        call, the others by the library after its up- and down-projection."""
        s = self.s
        with _span(timer, "route", stream):
            if s.router == "hash":
                if token_ids is None:
                    raise ValueError("the hash router needs token_ids")
                L.moe_route_hash(token_ids, s.E, s.k, s.salt, self.idx, self.gate, stream=stream)
            elif replay_idx is not None:
                self.idx.copy_(replay_idx)
                L.moe_route_replay(x, self.w_router, self.idx, s.score, self.logit_offset, self.gate, self.logits,
                                   stream=stream)
            else:
                L.moe_route(x, self.w_router, s.k, s.score, self.logit_offset, self.sel_bias,
                            self.idx, self.gate, self.logits, stream=stream)
        with _span(timer, "permute", stream):
            if s.capacity is None:
                L.moe_permute(self.idx, x, s.E, self.counts, self.offsets, self.row_of, self.token_of, self.x_perm,
                              workspace=self.ws_perm, stream=stream, copy=self.x_perm is not None)
            else:
                L.moe_permute_capacity(self.idx, x, s.E, s.capacity, self.counts, self.offsets, self.row_of,
                                       self.token_of, self.x_perm, workspace=self.ws_perm, stream=stream,
                                       copy=self.x_perm is not None)
        if ffn_events is not None:
            ffn_events[0].record(stream)
            L.moe_ffn_stage_events(ffn_events[1:])
        with _span(timer, "grouped_ffn", stream):
            if self.packed is not None:
                L.moe_grouped_ffn_packed(x if self.gather else self.x_perm, self.token_of if self.gather else None,
                                         self.offsets, *self.packed, s.f, self.gu, self.h, self.y_perm,
                                         workspace=self.ws_ffn, stream=stream)
            elif self.gather:
                L.moe_grouped_ffn_gather(x, self.token_of, self.offsets, self.w_gate_up, self.w_down, self.gu,
                                         self.h, self.y_perm, workspace=self.ws_ffn, stream=stream)
            else:
                L.moe_grouped_ffn(self.x_perm, self.offsets, self.w_gate_up, self.w_down, self.gu, self.h,
                                  self.y_perm, workspace=self.ws_ffn, stream=stream)
        shared_y = None
        if s.shared:
            with _span(timer, "shared_ffn", stream):
                if self.packed_sh is not None:
                    L.moe_grouped_ffn_packed(x, None, self.sh_offsets, *self.packed_sh, s.f_shared, self.sh_gu,
                                             self.sh_h, self.sh_y, workspace=self.ws_sh, stream=stream)
                else:
                    L.moe_grouped_ffn(x, self.sh_offsets, self.w_gate_up_shared, self.w_down_shared, self.sh_gu,
                                      self.sh_h, self.sh_y, workspace=self.ws_sh, stream=stream)
            shared_y = self.sh_y
        with _span(timer, "combine", stream):
            L.moe_combine(self.y_perm, self.row_of, self.gate, shared_y, self.out, stream=stream)
        if s.aux_alpha:
            with _span(timer, "aux_loss", stream):
                L.moe_aux_loss(self.logits, self.counts, s.k, s.score, s.aux_alpha, self.aux_loss, self.aux_p,
                               workspace=self.ws_aux, stream=stream)
        if s.bias_update and self.sel_bias is not None:
            with _span(timer, "bias_update", stream):
                L.moe_bias_update(self.sel_bias, self.counts, s.T, s.k, s.gamma, stream=stream)
        return self.out

    def backward(self, x, dy, stream=None, timer=None, stage_events=None):
        """Gradients of the last forward; stage_events as in _lib.moe_backward."""
        s = self.s
        a = L.BwdArgs()
        a.T, a.d, a.f, a.E, a.k = s.T, s.d, s.f, s.E, s.k
        a.score_fn = L.SCORE["uniform" if s.router == "hash" else s.score]
        for name, t in (("dy", dy), ("x", x), ("w_router", self.w_router), ("logits", self.logits),
                        ("topk_idx", self.idx), ("topk_gate", self.gate), ("row_of", self.row_of),
                        ("token_of", self.token_of), ("offsets", self.offsets), ("x_perm", self.x_perm),
                        ("gu_saved", self.gu), ("h", self.h), ("y_perm", self.y_perm),
                        ("w_gate_up", self.w_gate_up), ("w_down", self.w_down), ("dx", self.dx),
                        ("dw_router", self.dw_router), ("dw_gate_up", self.dw_gate_up), ("dw_down", self.dw_down),
                        ("dgate", self.dgate), ("dlogit", self.dlogit), ("workspace", self.ws_bwd)):
            setattr(a, name, t.data_ptr() if t is not None else None)
        a.workspace_bytes = self.ws_bwd.numel()
        a.counts = self.counts.data_ptr() if s.capacity is not None or s.aux_alpha else None
        a.aux_alpha = s.aux_alpha
        if s.shared:
            a.f_shared = s.f_shared
            for name, t in (("w_gate_up_shared", self.w_gate_up_shared[0]), ("w_down_shared", self.w_down_shared[0]),
                            ("gu_shared", self.sh_gu), ("h_shared", self.sh_h),
                            ("dw_gate_up_shared", self.dw_gate_up_shared), ("dw_down_shared", self.dw_down_shared),
                            ("workspace_shared", self.ws_bwd_sh)):
                setattr(a, name, t.data_ptr())
            a.workspace_shared_bytes = self.ws_bwd_sh.numel()
        with _span(timer, "backward", stream):
            L.moe_backward(a, stream=stream, stage_events=stage_events)
        return self.dx

    def capture(self, x, dy=None):
        """Record one step (forward, and the backward when dy is given) into a
        HIP graph; replaying it runs the same library kernels on the same
        buffers without per-call host work.  The library's calls allocate
        nothing and clear nothing with memset, so they can be captured."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward(x)
            if dy is not None:
                self.backward(x, dy)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x)
            if dy is not None:
                self.backward(x, dy)
        return g

