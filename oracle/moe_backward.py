"""Plain CPU oracle of the DeepSeekMoE layer backward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): shares no code with the
HIP library.

The pages train these layers (DeepSeek-V3 Technical Report summary, "3.2.1
DualPipe": each chunk runs attention and MLP forward and backward, the MLP
backward split into input and weight gradients); they print no formula for the
backward.  Reading: the backward is the gradient of the layer's forward
function (``moe_forward``) with the expert choice held fixed -- the top-K
selection is piecewise constant, so it has no gradient, and the selection bias
only chooses experts (DeepSeek-V3 summary, "2. Architecture": it is updated by
the load rule, not by gradients).  Gradients are those of the exact function:
fp64 throughout, scores computed in fp64 from fp64 logits.

For ``L = sum(dy * y)`` with ``y = x + sum_s FFN_s(x) + sum_k g_k FFN_{e_k}(x)``:

* an expert on rows u with output-side gradient dY: ``a1 = u W1^T``,
  ``a3 = u W3^T``, ``h = silu(a1) * a3``; ``dW2 = dY^T h``; ``dh = dY W2``;
  ``da1 = dh * a3 * silu'(a1)``, ``da3 = dh * silu(a1)``; ``dW1 = da1^T u``,
  ``dW3 = da3^T u``; ``du = da1 W1 + da3 W3``;
* shared experts see dY = dy; the k-th kept expert of token t sees
  ``dY = g_{t,k} dy_t``, and ``dg_{t,k} = dy_t . FFN_{e_k}(x_t)``;
* gate weights ``g_k = c s_{e_k}`` (c = routed_scale), or with renormalisation
  ``g_k = c s_{e_k} / S``, ``S = sum_k s_{e_k}``: ``ds_{e_k} = c dg_k`` or
  ``c (dg_k - sum_j dg_j g_j / c) / S``, zero at unchosen experts;
* scores: softmax ``dl = s * (ds - sum_e s_e ds_e)``; sigmoid
  ``dl = ds * s * (1 - s)``;
* logits ``l = x Wg^T + b``: ``dWg = dl^T x``, ``db = sum_t dl_t``,
  ``dx += dl Wg``; the residual adds ``dy`` to dx.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .moe_oracle import _as_expert_fn, route, silu


def dsilu(a: np.ndarray) -> np.ndarray:
    """d/da of a * sigmoid(a) = sigmoid(a) * (1 + a * (1 - sigmoid(a)))."""
    sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def expert_backward(u, dY, w1, w3, w2, magnitudes: bool = False):
    """One SwiGLU expert on rows ``u`` [R, d] with output gradient ``dY``
    [R, d].  Returns (du [R, d], dW1 [I, d], dW3 [I, d], dW2 [d, I], y [R, d]),
    fp64.  With ``magnitudes`` also the sums of the absolute values of the
    terms of du, dW1, dW3 and dW2 (same shapes): the scale of each result's
    rounding error when one factor of every term is rounded."""
    u = np.asarray(u, np.float64)
    dY = np.asarray(dY, np.float64)
    w1, w3, w2 = (np.asarray(w, np.float64) for w in (w1, w3, w2))
    a1 = u @ w1.T
    a3 = u @ w3.T
    h = silu(a1) * a3
    dW2 = dY.T @ h
    dh = dY @ w2
    da1 = dh * a3 * dsilu(a1)
    da3 = dh * silu(a1)
    out = (da1 @ w1 + da3 @ w3, da1.T @ u, da3.T @ u, dW2, h @ w2.T)
    if not magnitudes:
        return out
    A1, A3, U = np.abs(da1), np.abs(da3), np.abs(u)
    mag = (A1 @ np.abs(w1) + A3 @ np.abs(w3), A1.T @ U, A3.T @ U, np.abs(dY).T @ np.abs(h))
    return out + (mag,)


@dataclasses.dataclass
class Grads:
    dx: np.ndarray                  # [T, d]
    dw_gate: np.ndarray             # [E, d]
    dlogit_bias: np.ndarray         # [E]
    routed: tuple                   # (dW1 [E,I,d], dW3 [E,I,d], dW2 [E,d,I])
    shared: Optional[tuple]         # same for the K_s shared experts, or None
    dg: np.ndarray                  # [T, K] gradient of the gate weights
    dlogits: np.ndarray             # [T, E]
    idx: np.ndarray                 # [T, K] the expert choice used
    # with magnitudes=True: sums of |terms| of the experts' products (dx's
    # expert part; routed / shared (dW1, dW3, dW2)), else None
    dx_mag: Optional[np.ndarray] = None
    routed_mag: Optional[tuple] = None
    shared_mag: Optional[tuple] = None


def gate_weight_backward(s, idx, dg, norm_topk: bool, routed_scale: float):
    """ds [T, E] from dg [T, K] through g = c s_sel (or c s_sel / S)."""
    s = np.asarray(s, np.float64)
    T, E = s.shape
    c = float(routed_scale)
    s_sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    if norm_topk:
        S = s_sel.sum(axis=1, keepdims=True)
        w = s_sel / S                                   # the normalised weights
        ds_sel = c * (dg - (dg * w).sum(axis=1, keepdims=True)) / S
    else:
        ds_sel = c * dg
    ds = np.zeros((T, E))
    np.put_along_axis(ds, idx.astype(np.int64), ds_sel, axis=1)
    return ds


def score_backward(s, ds, score: str):
    """dl [T, E] from ds through softmax or sigmoid (s in fp64)."""
    s = np.asarray(s, np.float64)
    if score == "softmax":
        return s * (ds - (s * ds).sum(axis=1, keepdims=True))
    if score == "sigmoid":
        return ds * s * (1.0 - s)
    raise ValueError(f"unknown score function {score!r}")


def exact_scores(x, w_gate, logit_bias, score: str) -> np.ndarray:
    """Scores [T, E] in fp64 from fp64 logits (the differentiated function)."""
    l = np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T
    if logit_bias is not None:
        l = l + np.asarray(logit_bias, np.float64)[None, :]
    if score == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-l))


def moe_backward(x, w_gate, routed, shared, top_k: int, dy, *, n_shared: int = 0,
                 score: str = "softmax", logit_bias=None, select_bias=None,
                 n_groups: int = 1, topk_groups: int = 1, norm_topk: bool = False,
                 routed_scale: float = 1.0, forced_idx=None,
                 magnitudes: bool = False) -> Grads:
    """Gradients of ``sum(dy * y)`` for the layer forward of ``moe_forward``
    (same arguments), the expert choice held at the forward's (or
    ``forced_idx``).  ``magnitudes`` adds the sums of |terms| of the experts'
    products (see ``expert_backward``; routed terms weighted by |g|)."""
    x64 = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, d = x64.shape
    wg = np.asarray(w_gate, np.float64)
    E = wg.shape[0]
    r = route(x, w_gate, top_k, score=score, logit_bias=logit_bias,
              select_bias=select_bias, n_groups=n_groups, topk_groups=topk_groups,
              norm_topk=norm_topk, routed_scale=routed_scale, forced_idx=forced_idx)
    idx = r.idx.astype(np.int64)
    s = exact_scores(x, w_gate, logit_bias, score)
    s_sel = np.take_along_axis(s, idx, axis=1)
    g = s_sel / s_sel.sum(axis=1, keepdims=True) if norm_topk else s_sel
    g = g * float(routed_scale)

    dx = dy.copy()                                      # residual
    dx_mag = np.zeros((T, d)) if magnitudes else None
    shared_g = shared_m = None
    if n_shared > 0:
        fn = _as_expert_fn(shared)
        outs = [expert_backward(x64, dy, *fn(si), magnitudes=magnitudes)
                for si in range(n_shared)]
        for o in outs:
            dx += o[0]
        shared_g = tuple(np.stack([o[i] for o in outs]) for i in (1, 2, 3))
        if magnitudes:
            for o in outs:
                dx_mag += o[5][0]
            shared_m = tuple(np.stack([o[5][i] for o in outs]) for i in (1, 2, 3))

    fn = _as_expert_fn(routed)
    w1_0 = np.asarray(fn(0)[0])
    I = w1_0.shape[0]
    dW1 = np.zeros((E, I, d))
    dW3 = np.zeros((E, I, d))
    dW2 = np.zeros((E, d, I))
    dg = np.zeros((T, top_k))
    dx_routed = np.zeros((T, top_k, d))
    routed_m = tuple(np.zeros_like(a) for a in (dW1, dW3, dW2)) if magnitudes else None
    dx_routed_m = np.zeros((T, top_k, d)) if magnitudes else None
    for e in np.unique(idx):
        tt, kk = np.nonzero(idx == e)
        o = expert_backward(x64[tt], g[tt, kk, None] * dy[tt], *fn(int(e)),
                            magnitudes=magnitudes)
        du, d1, d3, d2, y_e = o[:5]
        dW1[e], dW3[e], dW2[e] = d1, d3, d2
        dx_routed[tt, kk] = du
        dg[tt, kk] = (dy[tt] * y_e).sum(axis=1)
        if magnitudes:
            dx_routed_m[tt, kk] = o[5][0]
            for j in range(3):
                routed_m[j][e] = o[5][j + 1]
    for k in range(top_k):
        dx += dx_routed[:, k]
        if magnitudes:
            dx_mag += dx_routed_m[:, k]

    ds = gate_weight_backward(s, idx, dg, norm_topk, routed_scale)
    dl = score_backward(s, ds, score)
    dx += dl @ wg
    return Grads(dx=dx, dw_gate=dl.T @ x64, dlogit_bias=dl.sum(axis=0),
                 routed=(dW1, dW3, dW2), shared=shared_g, dg=dg, dlogits=dl,
                 idx=r.idx, dx_mag=dx_mag, routed_mag=routed_m, shared_mag=shared_m)


def moe_forward_exact(x, w_gate, routed, shared, top_k: int, *, n_shared: int = 0,
                      score: str = "softmax", logit_bias=None, norm_topk: bool = False,
                      routed_scale: float = 1.0, forced_idx=None) -> np.ndarray:
    """The layer output in fp64 with fp64 scores and a given expert choice
    ``forced_idx`` [T, K] (the function ``moe_backward`` differentiates).
    Differs from ``moe_forward`` only in not rounding logits and scores to
    fp32."""
    x64 = np.asarray(x, np.float64)
    T, d = x64.shape
    idx = np.asarray(forced_idx, np.int64)
    s = exact_scores(x, w_gate, logit_bias, score)
    s_sel = np.take_along_axis(s, idx, axis=1)
    g = s_sel / s_sel.sum(axis=1, keepdims=True) if norm_topk else s_sel
    g = g * float(routed_scale)
    y = x64.copy()
    if n_shared > 0:
        fn = _as_expert_fn(shared)
        for si in range(n_shared):
            w1, w3, w2 = (np.asarray(w, np.float64) for w in fn(si))
            y += (silu(x64 @ w1.T) * (x64 @ w3.T)) @ w2.T
    fn = _as_expert_fn(routed)
    for t in range(T):
        for k in range(idx.shape[1]):
            w1, w3, w2 = (np.asarray(w, np.float64) for w in fn(int(idx[t, k])))
            u = x64[t]
            y[t] += g[t, k] * ((silu(w1 @ u) * (w3 @ u)) @ w2.T)
    return y
