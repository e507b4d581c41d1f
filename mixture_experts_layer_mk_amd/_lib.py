"""ctypes binding of ``libmoe_layer.so`` (C ABI in ``include/moe_layer.h``).

Argument marshalling only: shapes are read off the torch tensors, device
pointers and the current HIP stream are passed through, and every step of the
layer runs in the library's HIP kernels.  If the library has not been built
the binding raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_layer.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe_layer.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_WORKSPACE = -2
MOE_ERR_UNSUPPORTED = -3
MOE_ERR_ALIAS = -4
MOE_ERR_HIP = -5
MOE_ERR_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES

MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inner", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("shared_inner", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("score", ctypes.c_int32),
                ("norm_topk", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class FfnWeights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("s1", ctypes.c_void_p),
                ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class FfnGrads(ctypes.Structure):
    """moe_ffn_grads_t: fp32 weight gradients of a group of experts."""
    _fields_ = [("dw1", ctypes.c_void_p), ("dw3", ctypes.c_void_p), ("dw2", ctypes.c_void_p)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "topk_idx_i32", "topk_w_f32", "counts_i32", "offsets_i32",
        "slot_row_i32", "row_src_i32", "xp", "h_routed", "h_shared", "y", "y_scale_f32",
        "s_f32", "x_q", "x_scale", "h_routed_scale", "h_shared_scale", "total_bytes")]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def load_library():
    """Load the built library (raises RuntimeError if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_mk_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(MoeLayerDesc)
    lib.moe_layer_validate.argtypes = [D]
    lib.moe_layer_validate.restype = ctypes.c_int
    lib.moe_layer_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_layer_workspace_size.restype = ctypes.c_int
    lib.moe_layer_workspace_layout.argtypes = [D, ctypes.POINTER(WorkspaceLayout)]
    lib.moe_layer_workspace_layout.restype = ctypes.c_int
    fwd = [D, P, P, P, P, FfnWeights, FfnWeights, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_layer_forward.argtypes = fwd
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_layer_forward_noalloc.argtypes = fwd[:11] + [P]
    lib.moe_layer_forward_noalloc.restype = ctypes.c_int
    lib.moe_layer_forward_traced.argtypes = fwd + [ctypes.POINTER(P), ctypes.c_int32]
    lib.moe_layer_forward_traced.restype = ctypes.c_int
    lib.moe_layer_trace_stage_count.argtypes = []
    lib.moe_layer_trace_stage_count.restype = ctypes.c_int32
    lib.moe_layer_trace_stage_name.argtypes = [ctypes.c_int32]
    lib.moe_layer_trace_stage_name.restype = ctypes.c_char_p
    lib.moe_layer_backward_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_layer_backward_workspace_size.restype = ctypes.c_int
    lib.moe_layer_backward.argtypes = [D, P, P, P, P, FfnWeights, FfnWeights, P, P, P, P,
                                       FfnGrads, FfnGrads, P, P, ctypes.c_size_t, P]
    lib.moe_layer_backward.restype = ctypes.c_int
    lib.moe_layer_backward_traced.argtypes = lib.moe_layer_backward.argtypes + [
        ctypes.POINTER(P), ctypes.c_int32]
    lib.moe_layer_backward_traced.restype = ctypes.c_int
    lib.moe_layer_backward_stage_count.argtypes = []
    lib.moe_layer_backward_stage_count.restype = ctypes.c_int32
    lib.moe_layer_backward_stage_name.argtypes = [ctypes.c_int32]
    lib.moe_layer_backward_stage_name.restype = ctypes.c_char_p
    lib.moe_quantize_fp8_blocks.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, P, P, P]
    lib.moe_quantize_fp8_blocks.restype = ctypes.c_int
    lib.moe_bias_update.argtypes = [P, ctypes.c_int32, ctypes.c_float, P, P, P]
    lib.moe_bias_update.restype = ctypes.c_int
    lib.moe_side_stream_count.argtypes = []
    lib.moe_side_stream_count.restype = ctypes.c_int32
    lib.moe_strerror.argtypes = [ctypes.c_int]
    lib.moe_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions ``include/moe_layer.h`` declares."""
    import re
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def side_stream_count() -> int:
    """Side streams the library holds (one per host thread and device that ran
    an untraced forward or backward with shared experts; each is destroyed
    when its thread exits)."""
    return int(load_library().moe_side_stream_count())


def strerror(status: int) -> str:
    return load_library().moe_strerror(status).decode()


def make_desc(T, d, n_routed, top_k, inner, n_shared=0, shared_inner=0, *,
              n_groups=1, topk_groups=1, score="softmax", norm_topk=False,
              routed_scale=1.0, dtype="bf16") -> MoeLayerDesc:
    return MoeLayerDesc(
        T=T, d=d, n_routed=n_routed, top_k=top_k, inner=inner,
        n_shared=n_shared, shared_inner=shared_inner, n_groups=n_groups,
        topk_groups=topk_groups,
        score={"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}[score]
        if isinstance(score, str) else int(score),
        norm_topk=int(bool(norm_topk)), routed_scale=float(routed_scale),
        dtype={"bf16": MOE_BF16, "f32": MOE_F32, "fp8": MOE_FP8}[dtype]
        if isinstance(dtype, str) else int(dtype))


def validate(desc: Optional[MoeLayerDesc]) -> int:
    lib = load_library()
    return lib.moe_layer_validate(ctypes.byref(desc) if desc is not None else None)


def workspace_size(desc: MoeLayerDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().moe_layer_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return n.value


def workspace_layout(desc: MoeLayerDesc) -> dict:
    lay = WorkspaceLayout()
    st = load_library().moe_layer_workspace_layout(ctypes.byref(desc), ctypes.byref(lay))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return {n: getattr(lay, n) for n, _ in WorkspaceLayout._fields_}


def trace_stage_names() -> list:
    lib = load_library()
    return [lib.moe_layer_trace_stage_name(i).decode()
            for i in range(lib.moe_layer_trace_stage_count())]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, dtype, shape, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def backward_workspace_size(desc: MoeLayerDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().moe_layer_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return n.value


def backward_stage_names() -> list:
    lib = load_library()
    return [lib.moe_layer_backward_stage_name(i).decode()
            for i in range(lib.moe_layer_backward_stage_count())]


def moe_layer_backward(x, W_gate, experts: Sequence, shared: Optional[Sequence], K: int,
                       dout, *, score: str = "softmax", norm_topk: bool = False,
                       n_groups: int = 1, topk_groups: int = 1, select_bias=None,
                       logit_bias=None, routed_scale: float = 1.0, workspace=None,
                       stream=None, grads=None, trace_events=None):
    """Backward pass of the bf16 layer (``moe_layer_backward`` in the C ABI):
    gradients of sum(dout * out) for the forward on the same inputs, the
    expert choice held fixed.  Returns a dict: dx [T, d] bf16, dw_gate [E, d],
    dlogit_bias [E] (or None without a logit bias), routed = (dw1, dw3, dw2),
    shared = same or None (fp32), topk_idx [T, K] int32.  ``grads`` (a dict of
    that form) may be passed to write into existing tensors; ``trace_events``
    (n + 1 raw hipEvent_t handles, n = ``backward_stage_names()``) records
    every stage boundary."""
    import torch
    lib = load_library()
    dev = x.device
    if dev.type != "cuda" or x.dtype != torch.bfloat16:
        raise ValueError("x must be a bf16 GPU tensor")
    T, d = x.shape
    w1, w3, w2 = experts
    E, I = w1.shape[0], w1.shape[1]
    Ks, Is = (shared[0].shape[0], shared[0].shape[1]) if shared is not None else (0, 0)
    bf = torch.bfloat16
    _check_tensor("x", x, bf, (T, d), dev)
    _check_tensor("dout", dout, bf, (T, d), dev)
    _check_tensor("W_gate", W_gate, torch.float32, (E, d), dev)
    _check_tensor("experts.w1", w1, bf, (E, I, d), dev)
    _check_tensor("experts.w3", w3, bf, (E, I, d), dev)
    _check_tensor("experts.w2", w2, bf, (E, d, I), dev)
    if shared is not None:
        _check_tensor("shared.w1", shared[0], bf, (Ks, Is, d), dev)
        _check_tensor("shared.w3", shared[1], bf, (Ks, Is, d), dev)
        _check_tensor("shared.w2", shared[2], bf, (Ks, d, Is), dev)
    for name, b in (("select_bias", select_bias), ("logit_bias", logit_bias)):
        if b is not None:
            _check_tensor(name, b, torch.float32, (E,), dev)
    desc = make_desc(T, d, E, K, I, Ks, Is, n_groups=n_groups, topk_groups=topk_groups,
                     score=score, norm_topk=norm_topk, routed_scale=routed_scale,
                     dtype="bf16")
    st = lib.moe_layer_validate(ctypes.byref(desc))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    f32 = torch.float32
    if grads is None:
        grads = {
            "dx": torch.empty_like(x),
            "dw_gate": torch.empty((E, d), dtype=f32, device=dev),
            "dlogit_bias": torch.empty((E,), dtype=f32, device=dev) if logit_bias is not None
            else None,
            "routed": (torch.empty((E, I, d), dtype=f32, device=dev),
                       torch.empty((E, I, d), dtype=f32, device=dev),
                       torch.empty((E, d, I), dtype=f32, device=dev)),
            "shared": ((torch.empty((Ks, Is, d), dtype=f32, device=dev),
                        torch.empty((Ks, Is, d), dtype=f32, device=dev),
                        torch.empty((Ks, d, Is), dtype=f32, device=dev))
                       if shared is not None else None),
            "topk_idx": torch.empty((T, K), dtype=torch.int32, device=dev),
        }
    _check_tensor("dx", grads["dx"], bf, (T, d), dev)
    _check_tensor("dw_gate", grads["dw_gate"], f32, (E, d), dev)
    nbytes = backward_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ffn_r = FfnWeights(w1.data_ptr(), w3.data_ptr(), w2.data_ptr(), None, None, None)
    ffn_s = (FfnWeights(shared[0].data_ptr(), shared[1].data_ptr(), shared[2].data_ptr(),
                        None, None, None)
             if shared is not None else FfnWeights(None, None, None, None, None, None))
    gr = grads["routed"]
    for name, t, shp in (("dw1", gr[0], (E, I, d)), ("dw3", gr[1], (E, I, d)),
                         ("dw2", gr[2], (E, d, I))):
        _check_tensor("routed." + name, t, f32, shp, dev)
    g_r = FfnGrads(gr[0].data_ptr(), gr[1].data_ptr(), gr[2].data_ptr())
    if shared is not None:
        gs = grads["shared"]
        for name, t, shp in (("dw1", gs[0], (Ks, Is, d)), ("dw3", gs[1], (Ks, Is, d)),
                             ("dw2", gs[2], (Ks, d, Is))):
            _check_tensor("shared." + name, t, f32, shp, dev)
        g_s = FfnGrads(gs[0].data_ptr(), gs[1].data_ptr(), gs[2].data_ptr())
    else:
        g_s = FfnGrads(None, None, None)
    args = [ctypes.byref(desc), _ptr(x), _ptr(W_gate), _ptr(logit_bias), _ptr(select_bias),
            ffn_r, ffn_s, _ptr(dout), _ptr(grads["dx"]), _ptr(grads["dw_gate"]),
            _ptr(grads["dlogit_bias"]), g_r, g_s, _ptr(grads.get("topk_idx")),
            workspace.data_ptr(), workspace.numel(), stream]
    if trace_events is None:
        st = lib.moe_layer_backward(*args)
    else:
        arr = (ctypes.c_void_p * len(trace_events))(*trace_events)
        st = lib.moe_layer_backward_traced(*args, arr, len(trace_events))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return grads


def moe_layer_forward(x, W_gate, experts: Sequence, shared: Optional[Sequence],
                      K: int, *, score: str = "softmax", norm_topk: bool = False,
                      n_groups: int = 1, topk_groups: int = 1, select_bias=None,
                      logit_bias=None, routed_scale: float = 1.0,
                      return_routing: bool = False, out=None, workspace=None,
                      stream=None, trace_events=None, expert_scales=None,
                      shared_scales=None, _noalloc: bool = False):
    """DeepSeekMoE layer forward on the GPU.

    x [T, d] (bf16 or fp32), W_gate [E, d] fp32, experts = (w1 [E, I, d],
    w3 [E, I, d], w2 [E, d, I]), shared = same with K_s experts or None,
    K routed experts kept per token.  FP8 layer: x bf16, the weights uint8
    E4M3 codes and ``expert_scales`` / ``shared_scales`` = (s1 [E, I/128,
    d/128], s3 same, s2 [E, d/128, I/128]) uint8 block scale bytes (see
    ``quantize_fp8_blocks``).  Returns out [T, d] (and, with
    ``return_routing``, a dict with topk_idx [T, K] int32, topk_w [T, K] fp32
    and expert_counts [E] int32).  ``workspace`` (uint8, >= workspace_size)
    may be passed to reuse one buffer; ``trace_events`` (a list of n + 1 raw
    hipEvent_t handles) records every stage boundary."""
    import torch
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    dt = x.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {dt}")
    T, d = x.shape
    w1, w3, w2 = experts
    E, I = w1.shape[0], w1.shape[1]
    Ks, Is = (shared[0].shape[0], shared[0].shape[1]) if shared is not None else (0, 0)
    fp8 = expert_scales is not None
    if fp8 and dt != torch.bfloat16:
        raise ValueError("FP8 layers take bf16 x")
    wdt = torch.uint8 if fp8 else dt
    _check_tensor("x", x, dt, (T, d), dev)
    _check_tensor("W_gate", W_gate, torch.float32, (E, d), dev)
    _check_tensor("experts.w1", w1, wdt, (E, I, d), dev)
    _check_tensor("experts.w3", w3, wdt, (E, I, d), dev)
    _check_tensor("experts.w2", w2, wdt, (E, d, I), dev)
    if shared is not None:
        _check_tensor("shared.w1", shared[0], wdt, (Ks, Is, d), dev)
        _check_tensor("shared.w3", shared[1], wdt, (Ks, Is, d), dev)
        _check_tensor("shared.w2", shared[2], wdt, (Ks, d, Is), dev)
    if fp8:
        for name, sc, n, r, c in (("expert_scales", expert_scales, E, I, d),) + (
                (("shared_scales", shared_scales, Ks, Is, d),) if shared is not None else ()):
            if sc is None:
                raise ValueError(f"{name} required for an FP8 layer")
            _check_tensor(name + "[0]", sc[0], torch.uint8, (n, r // 128, c // 128), dev)
            _check_tensor(name + "[1]", sc[1], torch.uint8, (n, r // 128, c // 128), dev)
            _check_tensor(name + "[2]", sc[2], torch.uint8, (n, c // 128, r // 128), dev)
    for name, b in (("select_bias", select_bias), ("logit_bias", logit_bias)):
        if b is not None:
            _check_tensor(name, b, torch.float32, (E,), dev)
    desc = make_desc(T, d, E, K, I, Ks, Is, n_groups=n_groups,
                     topk_groups=topk_groups, score=score, norm_topk=norm_topk,
                     routed_scale=routed_scale,
                     dtype="fp8" if fp8 else "bf16" if dt == torch.bfloat16 else "f32")
    st = lib.moe_layer_validate(ctypes.byref(desc))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_tensor("out", out, dt, (T, d), dev)
    if _noalloc:
        if workspace is not None or trace_events is not None:
            raise ValueError("the no-allocation forward takes no workspace or trace events")
    else:
        nbytes = workspace_size(desc)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    idx = wts = cnt = None
    if return_routing:
        idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        wts = torch.empty((T, K), dtype=torch.float32, device=dev)
        cnt = torch.empty((E,), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    sr = tuple(t.data_ptr() for t in expert_scales) if fp8 else (None, None, None)
    ss = tuple(t.data_ptr() for t in shared_scales) if fp8 and shared is not None \
        else (None, None, None)
    ffn_r = FfnWeights(w1.data_ptr(), w3.data_ptr(), w2.data_ptr(), *sr)
    ffn_s = (FfnWeights(shared[0].data_ptr(), shared[1].data_ptr(), shared[2].data_ptr(), *ss)
             if shared is not None else FfnWeights(None, None, None, None, None, None))
    args = [ctypes.byref(desc), _ptr(x), _ptr(W_gate), _ptr(logit_bias),
            _ptr(select_bias), ffn_r, ffn_s, _ptr(out), _ptr(idx), _ptr(wts),
            _ptr(cnt)]
    if _noalloc:
        st = lib.moe_layer_forward_noalloc(*args, stream)
    elif trace_events is None:
        args += [workspace.data_ptr(), workspace.numel(), stream]
        st = lib.moe_layer_forward(*args)
    else:
        args += [workspace.data_ptr(), workspace.numel(), stream]
        arr = (ctypes.c_void_p * len(trace_events))(*trace_events)
        st = lib.moe_layer_forward_traced(*args, arr, len(trace_events))
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    if return_routing:
        return out, {"topk_idx": idx, "topk_w": wts, "expert_counts": cnt}
    return out


def moe_layer_forward_noalloc(x, W_gate, experts: Sequence, shared: Optional[Sequence],
                              K: int, **kw):
    """``moe_layer_forward`` through the C ABI's no-allocation entry point: the
    library's fixed per-device workspace (``MOE_NOALLOC_SCRATCH_BYTES``)
    instead of a caller's buffer, every stage in order on the stream.  Pass
    ``out=`` (and read routing with ``return_routing``) as for the allocating
    call; ``workspace`` and ``trace_events`` are not accepted.  Raises
    MoeError with MOE_ERR_SCRATCH when the layer does not fit."""
    return moe_layer_forward(x, W_gate, experts, shared, K, _noalloc=True, **kw)


def quantize_fp8_blocks(w, stream=None):
    """FP8 layer weight format: ``w`` [batch, rows, cols] (bf16 or fp32, GPU;
    rows, cols multiples of 128) to (E4M3 codes uint8 [batch, rows, cols],
    block scale bytes uint8 [batch, rows/128, cols/128])."""
    import torch
    lib = load_library()
    if w.device.type != "cuda" or not w.is_contiguous() or w.dim() != 3:
        raise ValueError("w must be a contiguous 3-d GPU tensor")
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {w.dtype}")
    B, R, C = w.shape
    codes = torch.empty((B, R, C), dtype=torch.uint8, device=w.device)
    scales = torch.empty((B, R // 128, C // 128), dtype=torch.uint8, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    st = lib.moe_quantize_fp8_blocks(w.data_ptr(), MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32,
                                     B, R, C, codes.data_ptr(), scales.data_ptr(), stream)
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return codes, scales


def moe_bias_update(counts, gamma: float, select_bias=None, rel_load=None, stream=None):
    """Auxiliary-loss-free bias update after a step: ``select_bias`` [E] fp32
    (updated in place, or None) moves by ``gamma`` down for overloaded and up
    for underloaded experts, judged from ``counts`` [E] int32 (e.g. the
    forward's expert_counts).  Returns the relative loads [E] fp32."""
    import torch
    lib = load_library()
    dev = counts.device
    if dev.type != "cuda":
        raise ValueError("counts must be a GPU tensor")
    E = counts.shape[0]
    _check_tensor("counts", counts, torch.int32, (E,), dev)
    if select_bias is not None:
        _check_tensor("select_bias", select_bias, torch.float32, (E,), dev)
    if rel_load is None:
        rel_load = torch.empty((E,), dtype=torch.float32, device=dev)
    else:
        _check_tensor("rel_load", rel_load, torch.float32, (E,), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.moe_bias_update(_ptr(counts), E, float(gamma), _ptr(select_bias),
                             _ptr(rel_load), stream)
    if st != MOE_OK:
        raise MoeError(st, strerror(st))
    return rel_load


class HipEvents:
    """A set of HIP events (hipEventCreate) for ``trace_events``, with
    elapsed-time queries.  Thin ctypes wrapper of the HIP runtime."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        self.hip.hipEventSynchronize(self.handles[j])
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i],
                                        self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self.hip.hipEventDestroy(h)
        self.handles = []
