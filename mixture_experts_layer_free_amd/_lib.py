"""ctypes binding of libmoe.so: the C ABI of include/moe.h, one Python function
per entry point, same names.  Argument marshalling only — every step runs in
the library's HIP kernels; torch supplies device memory and the stream.

The library must have been built (``python -m mixture_experts_layer_free_amd.build``);
loading fails loudly otherwise.  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
SCORE = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2, "uniform": 3}
(MOE_CALL_ROUTE, MOE_CALL_PERMUTE, MOE_CALL_GROUPED_FFN, MOE_CALL_BACKWARD, MOE_CALL_AUX_LOSS,
 MOE_CALL_BACKWARD_SHARED) = range(6)
# stages of moe_backward (enum moe_bwd_stage), in stream order
BWD_STAGES = ("combine", "dgrad_down", "router", "wgrad_down", "wgrad_up", "dgrad_up", "shared", "unpermute")
FFN_STAGES = ("up", "down")
MAX_EXPERTS, MAX_TOPK = 1024, 16
PERMUTE_NOALLOC_SCRATCH = 4 << 20   # bytes of moe_permute_noalloc's static device scratch

_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", _sz), ("T", _i64), ("d", _i64), ("f", _i64),
        ("E", _int), ("k", _int), ("score_fn", _int),
        ("dy", _vp), ("x", _vp), ("w_router", _vp), ("logits", _vp), ("topk_idx", _vp),
        ("topk_gate", _vp), ("row_of", _vp), ("token_of", _vp), ("offsets", _vp), ("x_perm", _vp),
        ("gu_saved", _vp), ("h", _vp), ("y_perm", _vp), ("w_gate_up", _vp), ("w_down", _vp),
        ("dx", _vp), ("dw_router", _vp), ("dw_gate_up", _vp), ("dw_down", _vp),
        ("dgate", _vp), ("dlogit", _vp),
        ("workspace", _vp), ("workspace_bytes", _sz),
        ("counts", _vp), ("aux_alpha", ctypes.c_float),
        ("f_shared", _i64), ("w_gate_up_shared", _vp), ("w_down_shared", _vp), ("gu_shared", _vp),
        ("h_shared", _vp), ("dw_gate_up_shared", _vp), ("dw_down_shared", _vp),
        ("workspace_shared", _vp), ("workspace_shared_bytes", _sz),
        ("stage_events", ctypes.POINTER(_vp)),
    ]


_SIGS = {
    "moe_route": [_vp, _int, _i64, _i64, _vp, _vp, _vp, _int, _int, _int, _vp, _vp, _vp, _vp],
    "moe_route_replay": [_vp, _int, _i64, _i64, _vp, _vp, _int, _int, _int, _vp, _vp, _vp, _vp],
    "moe_route_hash": [_vp, _i64, _int, _int, ctypes.c_uint32, _vp, _vp, _vp],
    "moe_permute": [_vp, _i64, _int, _int, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_permute_noalloc": [_vp, _i64, _int, _int, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_permute_capacity": [_vp, _i64, _int, _int, _i64, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_grouped_ffn": [_vp, _i64, _i64, _int, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_grouped_ffn_gather": [_vp, _i64, _vp, _i64, _i64, _int, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                               _vp],
    "moe_packed_weight_bytes": [_int, _i64, _i64, _i64],
    "moe_pack_expert_weights": [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "moe_grouped_ffn_packed": [_vp, _i64, _vp, _i64, _i64, _vp, _int, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "moe_ffn_stage_events": [ctypes.POINTER(_vp)],
    "moe_combine": [_vp, _vp, _vp, _vp, _i64, _int, _i64, _vp, _int, _vp],
    "moe_bias_update": [_vp, _vp, _int, _i64, _int, ctypes.c_float, _vp],
    "moe_aux_loss": [_vp, _vp, _i64, _int, _int, _int, ctypes.c_float, _vp, _vp, _vp, _sz, _vp],
    "moe_backward": [ctypes.POINTER(BwdArgs), _vp],
    "moe_workspace_size": [_int, _i64, _int, _int, _i64, _i64],
    "moe_status_str": [_int],
}

_lib = None


def lib():
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_free_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _int
        L.moe_workspace_size.restype = _sz
        L.moe_packed_weight_bytes.restype = _sz
        L.moe_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


class MoEError(RuntimeError):
    def __init__(self, name, status):
        super().__init__(f"{name} failed: {lib().moe_status_str(status).decode()} (status {status})")
        self.status = status


def _check(name, st):
    if st != MOE_OK:
        raise MoEError(name, st)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _out(t: Optional[torch.Tensor], name: str, dtype, shape, device) -> torch.Tensor:
    """A new output tensor, or the caller's after checking that the kernels
    can write it whole: a device tensor on the inputs' device, contiguous,
    with the expected dtype and shape."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _req(t, name, dtype, shape)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    return t


def workspace_size(which: int, T: int, k: int, E: int, d: int = 0, f: int = 0) -> int:
    return int(lib().moe_workspace_size(which, T, k, E, d, f))


def _workspace(which, T, k, E, d, f, device, workspace=None):
    """(workspace tensor, its size in bytes); a caller's workspace must be a
    contiguous device tensor on the inputs' device (the library checks its size)."""
    n = workspace_size(which, T, k, E, d, f)
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    else:
        _req(workspace, "workspace")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, the inputs on {device}")
    return workspace, workspace.numel() * workspace.element_size()


# ----------------------------------------------------------------------------
# entry points

def moe_route(x, w_router, k, score_fn, logit_offset=None, sel_bias=None,
              topk_idx=None, topk_gate=None, logits_out=None, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    _req(x, "x")
    _req(w_router, "w_router", torch.float32, (E, d))
    if logit_offset is not None:
        _req(logit_offset, "logit_offset", torch.float32, (E,))
    if sel_bias is not None:
        _req(sel_bias, "sel_bias", torch.float32, (E,))
    dev = x.device
    topk_idx = _out(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    topk_gate = _out(topk_gate, "topk_gate", torch.float32, (T, k), dev)
    logits_out = _out(logits_out, "logits_out", torch.float32, (T, E), dev)
    sf = SCORE[score_fn] if isinstance(score_fn, str) else int(score_fn)
    _check("moe_route", lib().moe_route(_p(x), _dtype_code(x), T, d, _p(w_router), _p(logit_offset),
                                        _p(sel_bias), E, k, sf, _p(topk_idx), _p(topk_gate),
                                        _p(logits_out), _stream(stream)))
    return topk_idx, topk_gate, logits_out


def moe_route_replay(x, w_router, topk_idx, score_fn, logit_offset=None, topk_gate=None, logits_out=None,
                     stream=None):
    """Logits and gates of the given expert choice topk_idx [T, k]."""
    T, d = x.shape
    E = w_router.shape[0]
    k = topk_idx.shape[1]
    _req(x, "x")
    _req(w_router, "w_router", torch.float32, (E, d))
    _req(topk_idx, "topk_idx", torch.int32, (T, k))
    if logit_offset is not None:
        _req(logit_offset, "logit_offset", torch.float32, (E,))
    dev = x.device
    topk_gate = _out(topk_gate, "topk_gate", torch.float32, (T, k), dev)
    logits_out = _out(logits_out, "logits_out", torch.float32, (T, E), dev)
    sf = SCORE[score_fn] if isinstance(score_fn, str) else int(score_fn)
    _check("moe_route_replay", lib().moe_route_replay(_p(x), _dtype_code(x), T, d, _p(w_router), _p(logit_offset),
                                                      E, k, sf, _p(topk_idx), _p(topk_gate), _p(logits_out),
                                                      _stream(stream)))
    return topk_gate, logits_out


def moe_route_hash(token_ids, E, k, salt=0, topk_idx=None, topk_gate=None, stream=None):
    """Hash router: the k experts with the smallest SplitMix64 keys, gates 1/k."""
    _req(token_ids, "token_ids", torch.int32)
    T = token_ids.shape[0]
    dev = token_ids.device
    topk_idx = _out(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    topk_gate = _out(topk_gate, "topk_gate", torch.float32, (T, k), dev)
    _check("moe_route_hash", lib().moe_route_hash(_p(token_ids), T, E, k, int(salt) & 0xFFFFFFFF, _p(topk_idx),
                                                  _p(topk_gate), _stream(stream)))
    return topk_idx, topk_gate


def moe_permute(topk_idx, x, E, counts=None, offsets=None, row_of=None, token_of=None, x_perm=None,
                workspace=None, stream=None, copy=True):
    """copy=False: indices only (x_perm is not written and comes back None)."""
    T, k = topk_idx.shape
    d = x.shape[1]
    _req(topk_idx, "topk_idx", torch.int32)
    _req(x, "x")
    dev = x.device
    A = T * k
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    row_of = _out(row_of, "row_of", torch.int32, (T, k), dev)
    token_of = _out(token_of, "token_of", torch.int32, (A,), dev)
    x_perm = _out(x_perm, "x_perm", x.dtype, (A, d), dev) if copy else None
    ws, n = _workspace(MOE_CALL_PERMUTE, T, k, E, d, 0, dev, workspace)
    if not copy:
        x_perm = None
    _check("moe_permute", lib().moe_permute(_p(topk_idx), T, k, E, _p(x), _dtype_code(x), d, _p(counts),
                                            _p(offsets), _p(row_of), _p(token_of), _p(x_perm), _p(ws),
                                            n, _stream(stream)))
    return counts, offsets, row_of, token_of, x_perm


def moe_permute_noalloc(topk_idx, x, E, counts=None, offsets=None, row_of=None, token_of=None, x_perm=None,
                        stream=None, copy=True):
    """moe_permute without a workspace: the library's static per-GPU scratch
    is used (calls that overlap on one GPU race).  Outputs a caller passes in
    are written in place; copy=False: indices only."""
    T, k = topk_idx.shape
    d = x.shape[1]
    _req(topk_idx, "topk_idx", torch.int32)
    _req(x, "x")
    dev = x.device
    A = T * k
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    row_of = _out(row_of, "row_of", torch.int32, (T, k), dev)
    token_of = _out(token_of, "token_of", torch.int32, (A,), dev)
    x_perm = _out(x_perm, "x_perm", x.dtype, (A, d), dev) if copy else None
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(_p(topk_idx), T, k, E, _p(x), _dtype_code(x), d,
                                                            _p(counts), _p(offsets), _p(row_of), _p(token_of),
                                                            _p(x_perm), _stream(stream)))
    return counts, offsets, row_of, token_of, x_perm


def moe_permute_capacity(topk_idx, x, E, capacity, counts=None, offsets=None, row_of=None, token_of=None,
                         x_perm=None, workspace=None, stream=None, copy=True):
    """moe_permute with an expert capacity in rows (< 0: none).  row_of holds ~r
    for a dropped assignment; offsets cover the kept rows.  copy=False: indices
    only."""
    T, k = topk_idx.shape
    d = x.shape[1]
    _req(topk_idx, "topk_idx", torch.int32)
    _req(x, "x")
    dev = x.device
    A = T * k
    counts = _out(counts, "counts", torch.int32, (E,), dev)
    offsets = _out(offsets, "offsets", torch.int32, (E + 1,), dev)
    row_of = _out(row_of, "row_of", torch.int32, (T, k), dev)
    token_of = _out(token_of, "token_of", torch.int32, (A,), dev)
    x_perm = _out(x_perm, "x_perm", x.dtype, (A, d), dev) if copy else None
    ws, n = _workspace(MOE_CALL_PERMUTE, T, k, E, d, 0, dev, workspace)
    if not copy:
        x_perm = None
    _check("moe_permute_capacity", lib().moe_permute_capacity(
        _p(topk_idx), T, k, E, int(capacity), _p(x), _dtype_code(x), d, _p(counts), _p(offsets), _p(row_of),
        _p(token_of), _p(x_perm), _p(ws), n, _stream(stream)))
    return counts, offsets, row_of, token_of, x_perm


def moe_grouped_ffn(x_rows, offsets, w_gate_up, w_down, gu_saved=None, h=None, y=None, save_gu=False,
                    workspace=None, stream=None):
    rows, d = x_rows.shape
    G = offsets.shape[0] - 1
    f = w_down.shape[2]
    _req(x_rows, "x_rows")
    _req(offsets, "offsets", torch.int32)
    _req(w_gate_up, "w_gate_up", x_rows.dtype, (G, 2 * f, d))
    _req(w_down, "w_down", x_rows.dtype, (G, d, f))
    dev = x_rows.device
    if save_gu or gu_saved is not None:
        gu_saved = _out(gu_saved, "gu_saved", x_rows.dtype, (rows, 2 * f), dev)
    h = _out(h, "h", x_rows.dtype, (rows, f), dev)
    y = _out(y, "y", torch.float32, (rows, d), dev)
    ws, n = _workspace(MOE_CALL_GROUPED_FFN, rows, 1, G, d, f, dev, workspace)
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(_p(x_rows), rows, d, _dtype_code(x_rows), _p(offsets), G, f,
                                                    _p(w_gate_up), _p(w_down), _p(gu_saved), _p(h), _p(y),
                                                    _p(ws), n, _stream(stream)))
    return gu_saved, h, y


def moe_grouped_ffn_gather(x, token_of, offsets, w_gate_up, w_down, gu_saved=None, h=None, y=None, save_gu=False,
                           workspace=None, stream=None):
    """moe_grouped_ffn on rows token_of[r] of x (the permute fused into the GEMM)."""
    T, d = x.shape
    rows = token_of.shape[0]
    G = offsets.shape[0] - 1
    f = w_down.shape[2]
    _req(x, "x")
    _req(token_of, "token_of", torch.int32, (rows,))
    _req(offsets, "offsets", torch.int32)
    _req(w_gate_up, "w_gate_up", x.dtype, (G, 2 * f, d))
    _req(w_down, "w_down", x.dtype, (G, d, f))
    dev = x.device
    if save_gu or gu_saved is not None:
        gu_saved = _out(gu_saved, "gu_saved", x.dtype, (rows, 2 * f), dev)
    h = _out(h, "h", x.dtype, (rows, f), dev)
    y = _out(y, "y", torch.float32, (rows, d), dev)
    ws, n = _workspace(MOE_CALL_GROUPED_FFN, rows, 1, G, d, f, dev, workspace)
    _check("moe_grouped_ffn_gather", lib().moe_grouped_ffn_gather(
        _p(x), T, _p(token_of), rows, d, _dtype_code(x), _p(offsets), G, f, _p(w_gate_up), _p(w_down),
        _p(gu_saved), _p(h), _p(y), _p(ws), n, _stream(stream)))
    return gu_saved, h, y


def packed_weight_bytes(which: int, G: int, d: int, f: int) -> int:
    return int(lib().moe_packed_weight_bytes(which, G, d, f))


def moe_pack_expert_weights(w_gate_up, w_down, packed_gate_up=None, packed_down=None, stream=None):
    """Tile-order copies of the expert weights for moe_grouped_ffn_packed
    (uint8 device tensors of moe_packed_weight_bytes; the layout is the
    library's own)."""
    G, f2, d = w_gate_up.shape
    f = f2 // 2
    _req(w_gate_up, "w_gate_up", torch.bfloat16)
    _req(w_down, "w_down", torch.bfloat16, (G, d, f))
    dev = w_gate_up.device
    packed_gate_up = _out(packed_gate_up, "packed_gate_up", torch.uint8, (packed_weight_bytes(0, G, d, f),), dev)
    packed_down = _out(packed_down, "packed_down", torch.uint8, (packed_weight_bytes(1, G, d, f),), dev)
    _check("moe_pack_expert_weights", lib().moe_pack_expert_weights(_p(w_gate_up), _p(w_down), G, d, f,
                                                                    _p(packed_gate_up), _p(packed_down),
                                                                    _stream(stream)))
    return packed_gate_up, packed_down


def moe_grouped_ffn_packed(x, token_of, offsets, packed_gate_up, packed_down, f, gu_saved=None, h=None, y=None,
                           save_gu=False, workspace=None, stream=None):
    """moe_grouped_ffn_gather (token_of given) or moe_grouped_ffn (token_of
    None: x holds the permuted rows) on weights from moe_pack_expert_weights."""
    T, d = x.shape
    rows = token_of.shape[0] if token_of is not None else T
    G = offsets.shape[0] - 1
    _req(x, "x", torch.bfloat16)
    if token_of is not None:
        _req(token_of, "token_of", torch.int32, (rows,))
    _req(offsets, "offsets", torch.int32)
    _req(packed_gate_up, "packed_gate_up", torch.uint8, (packed_weight_bytes(0, G, d, f),))
    _req(packed_down, "packed_down", torch.uint8, (packed_weight_bytes(1, G, d, f),))
    dev = x.device
    if save_gu or gu_saved is not None:
        gu_saved = _out(gu_saved, "gu_saved", x.dtype, (rows, 2 * f), dev)
    h = _out(h, "h", x.dtype, (rows, f), dev)
    y = _out(y, "y", torch.float32, (rows, d), dev)
    ws, n = _workspace(MOE_CALL_GROUPED_FFN, rows, 1, G, d, f, dev, workspace)
    _check("moe_grouped_ffn_packed", lib().moe_grouped_ffn_packed(
        _p(x), T, _p(token_of), rows, d, _p(offsets), G, f, _p(packed_gate_up), _p(packed_down),
        _p(gu_saved), _p(h), _p(y), _p(ws), n, _stream(stream)))
    return gu_saved, h, y


_ffn_events_keep = None   # the host array handed to the library, alive until the next setting


def moe_ffn_stage_events(events):
    """events: None, or len(FFN_STAGES) torch.cuda.Event objects, each
    recorded once before (so that it exists).  The next grouped FFN call on
    this thread records event s on its stream after stage s."""
    global _ffn_events_keep
    if events is None:
        _ffn_events_keep = None
        _check("moe_ffn_stage_events", lib().moe_ffn_stage_events(None))
        return
    if len(events) != len(FFN_STAGES):
        raise ValueError(f"moe_ffn_stage_events needs {len(FFN_STAGES)} events")
    _ffn_events_keep = (_vp * len(FFN_STAGES))(*[ev.cuda_event for ev in events])
    _check("moe_ffn_stage_events", lib().moe_ffn_stage_events(ctypes.cast(_ffn_events_keep, ctypes.POINTER(_vp))))


def moe_combine(y_perm, row_of, topk_gate, shared_y=None, out=None, out_dtype=torch.float32, stream=None):
    T, k = row_of.shape
    d = y_perm.shape[1]
    _req(y_perm, "y_perm", torch.float32, (T * k, d))
    _req(row_of, "row_of", torch.int32)
    _req(topk_gate, "topk_gate", torch.float32, (T, k))
    if shared_y is not None:
        _req(shared_y, "shared_y", torch.float32, (T, d))
    out = _out(out, "out", out_dtype if out is None else out.dtype, (T, d), y_perm.device)
    _check("moe_combine", lib().moe_combine(_p(y_perm), _p(row_of), _p(topk_gate), _p(shared_y), T, k, d,
                                            _p(out), _dtype_code(out), _stream(stream)))
    return out


def moe_bias_update(sel_bias, counts, T, k, gamma, stream=None):
    E = sel_bias.shape[0]
    _req(sel_bias, "sel_bias", torch.float32)
    _req(counts, "counts", torch.int32, (E,))
    _check("moe_bias_update", lib().moe_bias_update(_p(sel_bias), _p(counts), E, T, k, float(gamma),
                                                    _stream(stream)))
    return sel_bias


def moe_aux_loss(logits, counts, k, score_fn, alpha, loss_out=None, p_mean_out=None, workspace=None, stream=None):
    """Auxiliary load-balancing loss (device scalar) from the logits and counts."""
    T, E = logits.shape
    _req(logits, "logits", torch.float32)
    _req(counts, "counts", torch.int32, (E,))
    dev = logits.device
    loss_out = _out(loss_out, "loss_out", torch.float32, (1,), dev)
    if p_mean_out is not None:
        p_mean_out = _out(p_mean_out, "p_mean_out", torch.float32, (E,), dev)
    ws, n = _workspace(MOE_CALL_AUX_LOSS, T, k, E, 0, 0, dev, workspace)
    sf = SCORE[score_fn] if isinstance(score_fn, str) else int(score_fn)
    _check("moe_aux_loss", lib().moe_aux_loss(_p(logits), _p(counts), T, E, k, sf, float(alpha), _p(loss_out),
                                              _p(p_mean_out), _p(ws), n, _stream(stream)))
    return loss_out


def moe_backward(args: BwdArgs, stream=None, stage_events=None):
    """stage_events: None, or len(BWD_STAGES) torch.cuda.Event objects, each
    recorded once before (so that it exists); the library records event s on
    the stream after stage s."""
    args.struct_size = ctypes.sizeof(BwdArgs)
    keep = None
    if stage_events is not None:
        if len(stage_events) != len(BWD_STAGES):
            raise ValueError(f"stage_events needs {len(BWD_STAGES)} events")
        keep = (_vp * len(BWD_STAGES))(*[ev.cuda_event for ev in stage_events])
        args.stage_events = ctypes.cast(keep, ctypes.POINTER(_vp))
    else:
        args.stage_events = None
    _check("moe_backward", lib().moe_backward(ctypes.byref(args), _stream(stream)))
