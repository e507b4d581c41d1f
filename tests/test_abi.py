"""The C-ABI library loads, exports every function its header declares, and
rejects bad calls before touching the device (host-only checks; no kernel
runs here)."""
import ctypes

import pytest

import mixture_experts_layer_mk_amd as moe
from mixture_experts_layer_mk_amd import _lib

C16B = dict(T=16384, d=2048, n_routed=64, top_k=6, inner=1408, n_shared=2,
            shared_inner=1408)


def desc(**kw):
    p = dict(C16B)
    p.update(kw)
    extra = {k: p.pop(k) for k in list(p) if k in (
        "n_groups", "topk_groups", "score", "norm_topk", "routed_scale", "dtype")}
    return moe.make_desc(**p, **extra)


def test_library_exports_every_header_function():
    lib = moe.load_library()
    names = moe.header_functions()
    assert {"moe_layer_forward", "moe_layer_validate", "moe_layer_workspace_size",
            "moe_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_and_stage_names():
    for st in (moe.MOE_OK, moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_WORKSPACE,
               moe.MOE_ERR_UNSUPPORTED, moe.MOE_ERR_ALIAS, moe.MOE_ERR_HIP):
        assert moe.strerror(st) and moe.strerror(st) != "unknown status"
    names = moe.trace_stage_names()
    assert names == ["router", "scan", "permute", "gemm_gateup", "gemm_down", "combine"]


@pytest.mark.parametrize("kw,status", [
    (dict(), moe.MOE_OK),
    (dict(T=0), moe.MOE_OK),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=65), moe.MOE_ERR_INVALID_ARG),
    (dict(d=0), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, shared_inner=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=3), moe.MOE_ERR_INVALID_ARG),             # 64 % 3 != 0
    (dict(n_groups=8, topk_groups=9), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=8, topk_groups=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_groups=16, topk_groups=1), moe.MOE_ERR_INVALID_ARG),  # 4 < top_k
    (dict(score=2), moe.MOE_ERR_INVALID_ARG),
    (dict(routed_scale=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(n_routed=512, top_k=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_routed=64, top_k=40), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=2000), moe.MOE_ERR_UNSUPPORTED),                 # bf16 needs %64
    (dict(inner=1400), moe.MOE_ERR_UNSUPPORTED),
    (dict(dtype="f32", d=2000, inner=1400, shared_inner=1400), moe.MOE_OK),
    (dict(dtype="f32", d=2002), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=200000), moe.MOE_ERR_UNSUPPORTED),               # rows * d >= 2^31
    (dict(n_routed=256, top_k=8, n_groups=8, topk_groups=4, score="sigmoid",
          norm_topk=True), moe.MOE_OK),
])
def test_validate(kw, status):
    assert moe.validate(desc(**kw)) == status


def test_validate_null_and_raw_fields():
    assert moe.validate(None) == moe.MOE_ERR_INVALID_ARG
    d = desc()
    d.norm_topk = 2
    assert moe.validate(d) == moe.MOE_ERR_INVALID_ARG


def test_workspace_size_and_layout():
    d = desc()
    n = moe.workspace_size(d)
    lay = moe.workspace_layout(d)
    assert lay["total_bytes"] == n
    offs = [v for k, v in lay.items() if k != "total_bytes" and v >= 0]
    assert all(o % 256 == 0 for o in offs) and max(offs) < n
    TK = 16384 * 6
    assert lay["xp"] == -1          # token rows are gathered by the GEMM
    assert lay["y"] - lay["h_routed"] >= TK * 1408 * 2
    assert lay["y_scale_f32"] - lay["y"] >= TK * 2048 * 2     # fp16 routed outputs
    f32y = moe.workspace_layout(desc(dtype="f32"))
    assert f32y["y_scale_f32"] == -1                             # fp32 routed outputs
    # bf16 and FP8 with shared experts: S = x + shared experts (fp32) for the
    # separate combine after the side stream
    assert lay["s_f32"] >= 0 and lay["s_f32"] + 16384 * 2048 * 4 <= lay["total_bytes"]
    assert moe.workspace_layout(desc(dtype="fp8"))["s_f32"] >= 0
    f32 = moe.workspace_layout(desc(dtype="f32"))
    assert f32["s_f32"] >= 0 and f32["s_f32"] + 16384 * 2048 * 4 <= f32["total_bytes"]
    no_shared = moe.workspace_layout(desc(n_shared=0))
    assert no_shared["h_shared"] == -1 and no_shared["s_f32"] == -1
    assert moe.workspace_size(desc(n_shared=0)) < n
    with pytest.raises(moe.MoeError):
        moe.workspace_size(desc(top_k=0))


def _forward_raw(d, x, out, ws, ws_bytes, w=0x1000):
    lib = moe.load_library()
    P = ctypes.c_void_p
    ffn = _lib.FfnWeights(w, w, w)
    return lib.moe_layer_forward(ctypes.byref(d), x, w, None, None, ffn, ffn,
                                 out, None, None, None, ws, ws_bytes, None)


def test_forward_rejects_before_launch():
    """Every call here fails host-side validation, so no kernel is enqueued
    (the pointers are never dereferenced)."""
    d = desc()
    need = moe.workspace_size(d)
    fake_x, fake_out, fake_ws = 0x100000, 0x80000000, 0x40000000000
    # workspace too small / missing / misaligned
    assert _forward_raw(d, fake_x, fake_out, fake_ws, need - 1) == moe.MOE_ERR_WORKSPACE
    assert _forward_raw(d, fake_x, fake_out, None, need) == moe.MOE_ERR_WORKSPACE
    assert _forward_raw(d, fake_x, fake_out, fake_ws + 16, need) == moe.MOE_ERR_WORKSPACE
    # out aliases x (same pointer, and a partial overlap)
    assert _forward_raw(d, fake_x, fake_x, fake_ws, need) == moe.MOE_ERR_ALIAS
    assert _forward_raw(d, fake_x, fake_x + 4096, fake_ws, need) == moe.MOE_ERR_ALIAS
    # missing required pointers
    assert _forward_raw(d, None, fake_out, fake_ws, need) == moe.MOE_ERR_INVALID_ARG
    assert _forward_raw(d, fake_x, fake_out, fake_ws, need, w=0) == moe.MOE_ERR_INVALID_ARG
    # invalid descriptor
    assert _forward_raw(desc(top_k=0), fake_x, fake_out, fake_ws, need) == moe.MOE_ERR_INVALID_ARG
    lib = moe.load_library()
    ffn = _lib.FfnWeights(0x1000, 0x1000, 0x1000)
    assert lib.moe_layer_forward(None, fake_x, 0x1000, None, None, ffn, ffn, fake_out,
                                 None, None, None, fake_ws, need, None) == moe.MOE_ERR_INVALID_ARG
    # traced call needs stage count + 1 events
    ev = (ctypes.c_void_p * 3)(1, 2, 3)
    assert lib.moe_layer_forward_traced(
        ctypes.byref(d), fake_x, 0x1000, None, None, ffn, ffn, fake_out, None, None,
        None, fake_ws, need, None, ev, 3) == moe.MOE_ERR_INVALID_ARG


def test_python_binding_checks_tensors():
    import torch
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        moe.moe_layer_forward(x, torch.zeros(4, 64), (x, x, x), None, 2)
