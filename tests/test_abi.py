"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moe.h declares, and rejects bad arguments before
anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def built():
    from mixture_experts_layer_free_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_free_amd import build
        build.build()
    return _lib


@pytest.fixture(scope="module")
def L(built):
    """The binding, for argument checks that must fail before any launch.
    They pass a stand-in device pointer, so where a GPU is visible a call that
    unexpectedly passed its checks would launch on it: skipped there (the
    driver of these checks is the CPU suite)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only argument checks (stand-in pointers) are not run where a GPU is visible")
    return built


def test_exports_every_declared_entry_point(built):
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:moe_status|size_t|const char\*)\s+(moe_\w+)\s*\(", hdr, re.M)))
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_bias_update", "moe_backward",
            "moe_workspace_size", "moe_status_str"} <= set(names)
    lib = built.lib()
    for n in names:
        assert hasattr(lib, n), n


P = ctypes.c_void_p(4096)   # a non-null stand-in pointer: validation fails before it is ever used


def test_route_validation(L):
    lib = L.lib()
    args = lambda **kw: [kw.get("x", P), kw.get("dt", 1), kw.get("T", 64), kw.get("d", 64), P, None, None,
                         kw.get("E", 8), kw.get("k", 2), kw.get("sf", 0), P, P, kw.get("lo", P), None]
    assert lib.moe_route(*args(x=None)) == L.MOE_EINVAL
    assert lib.moe_route(*args(lo=None)) == L.MOE_EINVAL
    assert lib.moe_route(*args(k=9)) == L.MOE_EINVAL
    assert lib.moe_route(*args(k=0)) == L.MOE_EINVAL
    assert lib.moe_route(*args(T=0)) == L.MOE_EINVAL
    assert lib.moe_route(*args(sf=3)) == L.MOE_EINVAL
    assert lib.moe_route(*args(dt=7)) == L.MOE_EINVAL
    assert lib.moe_route(*args(E=1025, k=2)) == L.MOE_ENOTSUP
    assert lib.moe_route(*args(E=64, k=17)) == L.MOE_ENOTSUP
    assert lib.moe_route(*args(d=60)) == L.MOE_ENOTSUP
    assert lib.moe_route(*args(d=1 << 24)) == L.MOE_ENOTSUP   # 32-bit offsets within a 32-row tile


def test_permute_validation(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_PERMUTE, 1000, 8, 64)
    assert need >= 64 * ((8000 + 255) // 256) * 4
    a = lambda **kw: [P, kw.get("T", 1000), kw.get("k", 8), kw.get("E", 64), P, kw.get("dt", 1), kw.get("d", 64),
                      P, P, P, P, P, kw.get("ws", P), kw.get("wsb", need), None]
    assert lib.moe_permute(*a(ws=None)) == L.MOE_EWORKSPACE
    assert lib.moe_permute(*a(wsb=need - 1)) == L.MOE_EWORKSPACE
    assert lib.moe_permute(*a(k=65)) == L.MOE_EINVAL
    assert lib.moe_permute(*a(d=4)) == L.MOE_ENOTSUP        # 8-byte bf16 rows
    assert lib.moe_permute(*a(T=1 << 28, k=8, wsb=1 << 40)) == L.MOE_ENOTSUP   # T*k >= 2^31


def test_grouped_ffn_validation(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_GROUPED_FFN, 1000, 1, 64, 256, 128)
    a = lambda **kw: [P, 1000, kw.get("d", 256), kw.get("dt", 1), P, kw.get("G", 64), kw.get("f", 128), P, P,
                      None, kw.get("h", P), P, kw.get("ws", P), kw.get("wsb", need), None]
    assert lib.moe_grouped_ffn(*a(h=None)) == L.MOE_EINVAL
    assert lib.moe_grouped_ffn(*a(d=96)) == L.MOE_ENOTSUP
    assert lib.moe_grouped_ffn(*a(f=100)) == L.MOE_ENOTSUP
    assert lib.moe_grouped_ffn(*a(G=2000)) == L.MOE_ENOTSUP
    assert lib.moe_grouped_ffn(*a(wsb=0)) == L.MOE_EWORKSPACE
    assert lib.moe_grouped_ffn(*a(ws=None)) == L.MOE_EWORKSPACE
    # one expert's gate/up weight of 2 GiB: past one buffer resource
    assert lib.moe_grouped_ffn(*a(d=16384, f=32768)) == L.MOE_ENOTSUP
    assert lib.moe_grouped_ffn(*a(d=16384, f=32704, wsb=0)) == L.MOE_EWORKSPACE   # just under: the shape passes


def test_grouped_ffn_gather_validation(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_GROUPED_FFN, 512, 1, 4, 128, 128)
    a = lambda **kw: [P, kw.get("T", 256), kw.get("tok", P), 512, kw.get("d", 128), 1, P, 4, 128, P, P, None, P, P,
                      P, need, None]
    assert lib.moe_grouped_ffn_gather(*a(tok=None)) == L.MOE_EINVAL
    assert lib.moe_grouped_ffn_gather(*a(T=0)) == L.MOE_EINVAL
    assert lib.moe_grouped_ffn_gather(*a(d=96)) == L.MOE_ENOTSUP
    assert lib.moe_grouped_ffn_gather(*a(T=1 << 23, d=128)) == L.MOE_ENOTSUP   # x past one buffer resource


def test_ffn_stage_events_setting(L):
    """The timing hook takes a host array (or NULL) and returns OK; a grouped
    FFN call that fails its checks takes the setting and records nothing."""
    lib = L.lib()
    lib.moe_ffn_stage_events.restype = ctypes.c_int
    arr = (ctypes.c_void_p * 2)(None, None)
    assert lib.moe_ffn_stage_events(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))) == L.MOE_OK
    need = L.workspace_size(L.MOE_CALL_GROUPED_FFN, 1000, 1, 64, 256, 128)
    assert lib.moe_grouped_ffn(P, 1000, 256, 1, P, 64, 128, P, P, None, None, P, P, need, None) == L.MOE_EINVAL
    assert lib.moe_ffn_stage_events(None) == L.MOE_OK


def test_permute_without_copy_needs_no_x(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_PERMUTE, 1000, 8, 64)
    # a copy needs x; indices only do not (that call would enqueue, so only the rejection is exercised here)
    assert lib.moe_permute(P, 1000, 8, 64, None, 1, 64, P, P, P, P, P, P, need, None) == L.MOE_EINVAL


def test_packed_weight_calls(L):
    """The packed-weight entry points: sizes of the packed copies, and the
    argument checks of packing and of the packed grouped FFN."""
    lib = L.lib()
    assert L.packed_weight_bytes(0, 3, 192, 256) == 3 * 512 * 192 * 2       # gate/up: the same bytes
    assert L.packed_weight_bytes(1, 3, 192, 256) == 3 * 256 * 256 * 2       # down: rows padded to 256
    assert L.packed_weight_bytes(1, 2, 512, 128) == 2 * 512 * 128 * 2
    assert L.packed_weight_bytes(2, 3, 192, 256) == 0 and L.packed_weight_bytes(0, 0, 192, 256) == 0
    pack = lambda **kw: lib.moe_pack_expert_weights(kw.get("gu", P), P, kw.get("G", 4), kw.get("d", 256),
                                                    kw.get("f", 256), kw.get("pgu", P), P, None)
    assert pack(gu=None) == L.MOE_EINVAL
    assert pack(pgu=None) == L.MOE_EINVAL
    assert pack(G=0) == L.MOE_EINVAL
    assert pack(d=96) == L.MOE_ENOTSUP
    assert pack(f=192) == L.MOE_ENOTSUP          # the 256 x 256 tile needs f % 128 == 0
    assert pack(G=2000) == L.MOE_ENOTSUP
    need = L.workspace_size(L.MOE_CALL_GROUPED_FFN, 1000, 1, 64, 256, 256)
    ffn = lambda **kw: lib.moe_grouped_ffn_packed(kw.get("x", P), 1000, kw.get("tok", P), 1000, kw.get("d", 256), P,
                                                  64, kw.get("f", 256), P, P, None, P, P, kw.get("ws", P),
                                                  kw.get("wsb", need), None)
    assert ffn(f=192) == L.MOE_ENOTSUP
    assert ffn(x=None) == L.MOE_EINVAL
    assert ffn(d=96) == L.MOE_ENOTSUP
    assert ffn(wsb=0) == L.MOE_EWORKSPACE


def test_combine_and_bias_validation(L):
    lib = L.lib()
    assert lib.moe_combine(None, P, P, None, 10, 2, 64, P, 0, None) == L.MOE_EINVAL
    assert lib.moe_combine(P, P, P, None, 10, 17, 64, P, 0, None) == L.MOE_ENOTSUP
    assert lib.moe_combine(P, P, P, None, 10, 2, 66, P, 0, None) == L.MOE_ENOTSUP
    assert lib.moe_combine(P, P, P, None, 10, 2, 64, P, 5, None) == L.MOE_EINVAL
    assert lib.moe_bias_update(None, P, 8, 64, 2, 1e-3, None) == L.MOE_EINVAL
    assert lib.moe_bias_update(P, P, 8, 64, 9, 1e-3, None) == L.MOE_EINVAL


def test_route_variants_validation(L):
    lib = L.lib()
    # moe_route_replay: the score function must be a learned one
    r = lambda **kw: [P, 1, kw.get("T", 64), kw.get("d", 64), P, None, kw.get("E", 8), kw.get("k", 2),
                      kw.get("sf", 0), kw.get("idx", P), P, P, None]
    assert lib.moe_route_replay(*r(idx=None)) == L.MOE_EINVAL
    assert lib.moe_route_replay(*r(sf=3)) == L.MOE_EINVAL
    assert lib.moe_route_replay(*r(d=12)) == L.MOE_ENOTSUP
    assert lib.moe_route_replay(*r(E=2048)) == L.MOE_ENOTSUP
    # moe_route_hash
    assert lib.moe_route_hash(None, 64, 8, 2, 0, P, P, None) == L.MOE_EINVAL
    assert lib.moe_route_hash(P, 64, 8, 9, 0, P, P, None) == L.MOE_EINVAL
    assert lib.moe_route_hash(P, 64, 64, 17, 0, P, P, None) == L.MOE_ENOTSUP
    assert lib.moe_route_hash(P, 1 << 31, 8, 2, 0, P, P, None) == L.MOE_ENOTSUP


def test_permute_capacity_validation(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_PERMUTE, 1000, 8, 64)
    a = lambda **kw: [P, 1000, kw.get("k", 8), 64, kw.get("cap", 200), P, 1, kw.get("d", 64), P, P,
                      kw.get("row_of", P), P, P, P, kw.get("wsb", need), None]
    assert lib.moe_permute_capacity(*a(row_of=None)) == L.MOE_EINVAL
    assert lib.moe_permute_capacity(*a(k=65)) == L.MOE_EINVAL
    assert lib.moe_permute_capacity(*a(d=4)) == L.MOE_ENOTSUP
    assert lib.moe_permute_capacity(*a(wsb=need - 1)) == L.MOE_EWORKSPACE


def test_aux_loss_validation(L):
    lib = L.lib()
    need = L.workspace_size(L.MOE_CALL_AUX_LOSS, 1000, 8, 64)
    a = lambda **kw: [kw.get("lg", P), P, kw.get("T", 1000), kw.get("E", 64), kw.get("k", 8), kw.get("sf", 1),
                      0.01, P, None, P, kw.get("wsb", need), None]
    assert need > 0
    assert lib.moe_aux_loss(*a(lg=None)) == L.MOE_EINVAL
    assert lib.moe_aux_loss(*a(k=65)) == L.MOE_EINVAL
    assert lib.moe_aux_loss(*a(sf=3)) == L.MOE_EINVAL      # hash routing has no router probabilities
    assert lib.moe_aux_loss(*a(E=2048, k=8)) == L.MOE_ENOTSUP
    assert lib.moe_aux_loss(*a(wsb=need - 1)) == L.MOE_EWORKSPACE


def _bwd_args(L, **kw):
    a = L.BwdArgs()
    a.struct_size = kw.get("struct_size", ctypes.sizeof(L.BwdArgs))
    a.T, a.d, a.f = kw.get("T", 1000), kw.get("d", 256), kw.get("f", 128)
    a.E, a.k, a.score_fn = kw.get("E", 64), kw.get("k", 8), kw.get("score_fn", 2)
    for name in ("dy", "x", "w_router", "logits", "topk_idx", "topk_gate", "row_of", "token_of", "offsets",
                 "x_perm", "gu_saved", "h", "y_perm", "w_gate_up", "w_down", "dx", "dw_router", "dw_gate_up",
                 "dw_down", "workspace"):
        setattr(a, name, kw.get(name, P.value))
    a.workspace_bytes = kw.get("workspace_bytes", L.workspace_size(L.MOE_CALL_BACKWARD, a.T, a.k, a.E, a.d, a.f))
    a.counts = kw.get("counts", None)
    a.aux_alpha = kw.get("aux_alpha", 0.0)
    if kw.get("shared"):
        a.f_shared = kw.get("f_shared", 128)
        for name in ("w_gate_up_shared", "w_down_shared", "gu_shared", "h_shared", "dw_gate_up_shared",
                     "dw_down_shared", "workspace_shared"):
            setattr(a, name, kw.get(name, P.value))
        a.workspace_shared_bytes = kw.get("workspace_shared_bytes", L.workspace_size(
            L.MOE_CALL_BACKWARD_SHARED, a.T, 1, 1, a.d, a.f_shared))
    return a


def test_backward_validation(L):
    lib = L.lib()
    bwd = lambda **kw: lib.moe_backward(ctypes.byref(_bwd_args(L, **kw)), None)
    assert bwd(struct_size=8) == L.MOE_EINVAL
    assert bwd(k=65) == L.MOE_EINVAL
    assert bwd(score_fn=4) == L.MOE_EINVAL
    assert bwd(dy=None) == L.MOE_EINVAL
    assert bwd(w_router=None) == L.MOE_EINVAL                     # a learned router needs its weight
    assert bwd(aux_alpha=0.01) == L.MOE_EINVAL                    # the aux gradient needs the counts
    assert bwd(score_fn=3, aux_alpha=0.01, counts=P.value) == L.MOE_EINVAL   # and a learned router
    assert bwd(d=96) == L.MOE_ENOTSUP
    assert bwd(x_perm=None, d=96) == L.MOE_ENOTSUP                # x_perm may be NULL (x is read through token_of)
    assert bwd(x_perm=None, x=None) == L.MOE_EINVAL               # x may not
    assert bwd(y_perm=None, workspace_bytes=0) == L.MOE_EWORKSPACE   # y_perm is not read
    assert bwd(f=100) == L.MOE_ENOTSUP
    assert bwd(E=2048, k=8) == L.MOE_ENOTSUP
    assert bwd(T=1 << 20, d=1024, workspace_bytes=1 << 50) == L.MOE_ENOTSUP   # X_perm past 2 GiB
    assert bwd(workspace_bytes=0) == L.MOE_EWORKSPACE
    assert bwd(workspace=None) == L.MOE_EWORKSPACE
    # an older caller's struct, ending before an appended field, passes the size check
    for field in ("counts", "aux_alpha", "f_shared", "stage_events"):
        assert bwd(struct_size=getattr(L.BwdArgs, field).offset, workspace_bytes=0) == L.MOE_EWORKSPACE, field
    assert bwd(struct_size=L.BwdArgs.f_shared.offset + 8) == L.MOE_EINVAL
    # the shared expert's fields
    assert bwd(shared=True, h_shared=None) == L.MOE_EINVAL
    assert bwd(shared=True, f_shared=0) == L.MOE_EINVAL
    assert bwd(shared=True, f_shared=96) == L.MOE_ENOTSUP
    assert bwd(shared=True, workspace_shared=None) == L.MOE_EWORKSPACE
    assert bwd(shared=True, workspace_shared_bytes=1) == L.MOE_EWORKSPACE
    # an older caller's struct ending before f_shared ignores the shared fields
    assert bwd(shared=True, f_shared=96, struct_size=L.BwdArgs.f_shared.offset, workspace_bytes=0) == \
        L.MOE_EWORKSPACE


def test_backward_shared_workspace_size(built):
    """The shared expert's backward workspace: dG|dU (bf16) and its input
    gradient (f32) over T rows, the weight gradients' chunk schedule, and
    their per-chunk partial outputs: at most 2*ceil(T/512) chunks of the
    larger weight gradient (chunks hold at least 512 rows)."""
    T, d, fs = 1000, 256, 128
    n = built.workspace_size(built.MOE_CALL_BACKWARD_SHARED, T, 1, 1, d, fs)
    base = T * 2 * fs * 2 + T * d * 4
    assert n >= base
    assert n <= base + 2 * -(-T // 512) * (2 * fs * d * 4) + 65536


def test_status_strings(L):
    lib = L.lib()
    assert lib.moe_status_str(0) == b"ok"
    assert b"workspace" in lib.moe_status_str(3)
    assert lib.moe_status_str(99) == b"unknown status"
