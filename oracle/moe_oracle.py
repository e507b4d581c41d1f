"""Plain CPU oracle of the DeepSeekMoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module: only the tests, the package smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes (one token ``u_t`` of hidden size d; mN routed experts, mK
kept, K_s shared experts; DeepSeekMoE paper abstract, and the DeepSeekMoE blog
post sections "Fine-Grained Expert Segmentation (Section 3.1)" and "Shared
Expert Isolation (Section 3.2)"):

1. affinity logits ``l_{t,e} = u_t . w_e (+ logit_bias_e)`` for every routed
   expert e (gate vectors ``w_e``);
2. scores ``s = softmax(l)`` over the routed experts, or ``s = sigmoid(l)``
   for the V3-style layer;
3. selection keys ``key = s (+ select_bias)`` -- the bias only chooses
   experts and never scales them (DeepSeek-V3 Technical Report summary,
   "2. Architecture", auxiliary-loss-free load balancing);
4. optional group limit: experts are split into contiguous groups; each group
   is ranked by the sum of its two highest keys and only the best groups stay
   eligible (same section, node-limited routing, read on one GPU as
   group-limited routing);
5. keep the mK largest keys, ordered by key descending then expert index
   ascending; no token is ever dropped (same section);
6. gate weights ``g = s`` at the kept experts, optionally renormalised to sum
   to one, times ``routed_scale``;
7. ``y_t = u_t + sum_s FFN_shared_s(u_t) + sum_k g_{t,k} FFN_{sel_k}(u_t)``,
   with every expert a SwiGLU FFN ``W2 (silu(W1 u) * (W3 u))`` and the shared
   experts always active with weight one (blog post, "DeepSeekMoE 2B Model
   Example").

Precision.  Outputs are computed in fp64 from the exact input values.  The
routing decision (an integer chosen by floating point) is taken in fp32, the
precision the GPU router decides in: logits are the fp64 dot products rounded
once to fp32, biases are added in fp32, scores are the fp64 softmax/sigmoid of
those fp32 logits rounded once to fp32, and keys, group sums and the top-K
comparisons are fp32.  The margins returned with the routing say how far each
decision is from a tie.

Every function here is pinned by a test under ``tests/`` that checks it
against something other than itself (closed forms, brute force, invariants,
the pages' own parameter counts).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Sequence

import numpy as np

ExpertFn = Callable[[int], tuple]   # e -> (w1 [I,d], w3 [I,d], w2 [d,I])


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Routing:
    idx: np.ndarray           # [T, K] int32, key descending then index ascending
    g: np.ndarray             # [T, K] fp64 gate weights of the kept experts
    scores: np.ndarray        # [T, E] fp32 s (softmax or sigmoid)
    keys: np.ndarray          # [T, E] fp32 selection keys (masked: -inf)
    margin: np.ndarray        # [T] fp64 key_(K) - key_(K+1)   (inf if none)
    group_margin: np.ndarray  # [T] fp64 G_(kept) - G_(kept+1) (inf if no groups)


def gate_logits(x, w_gate, logit_bias=None) -> np.ndarray:
    """Affinity logits [T, E] in fp32: fp64 dot products rounded once, then
    the optional logit bias added in fp32."""
    l64 = np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T
    l32 = l64.astype(np.float32)
    if logit_bias is not None:
        l32 = l32 + np.asarray(logit_bias, np.float32)[None, :]
    return l32


def gate_scores(l32: np.ndarray, score: str) -> np.ndarray:
    """Token-to-expert scores [T, E] in fp32 (fp64 math, one rounding)."""
    l = l32.astype(np.float64)
    if score == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        s = z / z.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-l))
    else:
        raise ValueError(f"unknown score function {score!r}")
    return s.astype(np.float32)


def _order_desc(v: np.ndarray) -> np.ndarray:
    """Column order of each row of v: value descending, then index ascending.
    (A stable sort of -v keeps equal values in index order.)"""
    return np.argsort(-v, axis=1, kind="stable")


def group_scores(keys: np.ndarray, n_groups: int) -> np.ndarray:
    """Score of each contiguous expert group: the fp32 sum of its two highest
    keys (one key if a group holds a single expert).  [T, n_groups] fp32."""
    T, E = keys.shape
    gs = E // n_groups
    kg = keys.reshape(T, n_groups, gs)
    top = -np.sort(-kg, axis=2)           # descending within each group
    if gs == 1:
        return top[:, :, 0].astype(np.float32)
    return (top[:, :, 0] + top[:, :, 1]).astype(np.float32)   # fp32 add


def select_experts(scores: np.ndarray, top_k: int, select_bias=None,
                   n_groups: int = 1, topk_groups: int = 1):
    """Top-K choice on fp32 keys; returns (idx, keys_masked, margin,
    group_margin)."""
    T, E = scores.shape
    keys = scores.astype(np.float32)
    if select_bias is not None:
        keys = keys + np.asarray(select_bias, np.float32)[None, :]
    group_margin = np.full(T, np.inf)
    if n_groups > 1:
        G = group_scores(keys, n_groups)
        gord = _order_desc(G)
        kept = gord[:, :topk_groups]
        if topk_groups < n_groups:
            Gs = np.take_along_axis(G, gord, axis=1).astype(np.float64)
            group_margin = Gs[:, topk_groups - 1] - Gs[:, topk_groups]
        allowed = np.zeros((T, n_groups), bool)
        np.put_along_axis(allowed, kept, True, axis=1)
        allowed_e = np.repeat(allowed, E // n_groups, axis=1)
        keys = np.where(allowed_e, keys, np.float32(-np.inf)).astype(np.float32)
    order = _order_desc(keys)
    idx = order[:, :top_k].astype(np.int32)
    ks = np.take_along_axis(keys, order, axis=1).astype(np.float64)
    if top_k < E:
        with np.errstate(invalid="ignore"):
            margin = ks[:, top_k - 1] - ks[:, top_k]
        margin = np.where(np.isneginf(ks[:, top_k]), np.inf, margin)
    else:
        margin = np.full(T, np.inf)
    return idx, keys, margin, group_margin


def route(x, w_gate, top_k: int, *, score: str = "softmax", logit_bias=None,
          select_bias=None, n_groups: int = 1, topk_groups: int = 1,
          norm_topk: bool = False, routed_scale: float = 1.0,
          forced_idx: Optional[np.ndarray] = None) -> Routing:
    """Gate, select and weight (steps 1-6 of the module docstring).

    ``forced_idx`` replaces the choice (used where a token sits within the
    tie tolerance and another valid choice was made); weights are then the
    oracle's scores at the forced experts."""
    l32 = gate_logits(x, w_gate, logit_bias)
    s = gate_scores(l32, score)
    idx, keys, margin, gmargin = select_experts(s, top_k, select_bias,
                                                n_groups, topk_groups)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, np.int32)
    g = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    if norm_topk:
        g = g / g.sum(axis=1, keepdims=True)
    g = g * float(routed_scale)
    return Routing(idx=idx, g=g, scores=s, keys=keys, margin=margin,
                   group_margin=gmargin)


# ---------------------------------------------------------------------------
# Experts and the layer
# ---------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """SiLU a * sigmoid(a) in fp64."""
    return a / (1.0 + np.exp(-a))


def swiglu_ffn(u: np.ndarray, w1, w3, w2) -> np.ndarray:
    """One expert: ``W2 (silu(W1 u) * (W3 u))`` for every row u of ``u``.

    w1, w3: [inner, d]; w2: [d, inner] (output-major, like a linear layer's
    weight).  fp64."""
    u = np.asarray(u, np.float64)
    a = u @ np.asarray(w1, np.float64).T
    b = u @ np.asarray(w3, np.float64).T
    h = silu(a) * b
    return h @ np.asarray(w2, np.float64).T


def _as_expert_fn(experts) -> ExpertFn:
    if experts is None:
        return None
    if callable(experts):
        return experts
    if isinstance(experts, (tuple, list)) and len(experts) == 3 and \
            getattr(experts[0], "ndim", 0) == 3:
        w1, w3, w2 = experts
        return lambda e: (w1[e], w3[e], w2[e])
    return lambda e: experts[e]


def moe_forward(x, w_gate, routed, shared, top_k: int, *, n_shared: int = 0,
                score: str = "softmax", logit_bias=None, select_bias=None,
                n_groups: int = 1, topk_groups: int = 1,
                norm_topk: bool = False, routed_scale: float = 1.0,
                forced_idx=None, stats: Optional[dict] = None):
    """The layer forward (steps 1-7).  Returns (y [T, d] fp64, Routing).

    ``routed`` / ``shared``: stacked (w1 [E,I,d], w3 [E,I,d], w2 [E,d,I]) or a
    callable ``e -> (w1, w3, w2)``.  Sums are taken in the order of the
    definition: residual, shared experts in index order, then the kept
    routed experts in key order k = 0..K-1.  ``stats`` (optional dict)
    receives the multiply-add count actually performed."""
    x64 = np.asarray(x, np.float64)
    T, d = x64.shape
    r = route(x, w_gate, top_k, score=score, logit_bias=logit_bias,
              select_bias=select_bias, n_groups=n_groups,
              topk_groups=topk_groups, norm_topk=norm_topk,
              routed_scale=routed_scale, forced_idx=forced_idx)
    macs = T * d * np.asarray(w_gate).shape[0]
    y = x64.copy()
    shared_fn = _as_expert_fn(shared)
    for s_i in range(n_shared):
        w1, w3, w2 = shared_fn(s_i)
        y += swiglu_ffn(x64, w1, w3, w2)
        macs += T * 3 * d * np.asarray(w1).shape[0]
    # Each kept expert's FFN output for each (token, slot); every expert's
    # weights are fetched once, for all rows that chose it.
    routed_fn = _as_expert_fn(routed)
    contrib = np.zeros((T, top_k, d))
    for e in np.unique(r.idx):
        tt, kk = np.nonzero(r.idx == e)
        w1, w3, w2 = routed_fn(int(e))
        contrib[tt, kk] = swiglu_ffn(x64[tt], w1, w3, w2)
        macs += tt.size * 3 * d * np.asarray(w1).shape[0]
    for k in range(top_k):
        y += r.g[:, k, None] * contrib[:, k]
    if stats is not None:
        stats["macs"] = int(macs)
    return y, r


def moe_forward_bruteforce(x, w_gate, routed, shared, top_k: int, *,
                           n_shared: int = 0, score: str = "softmax",
                           logit_bias=None, select_bias=None,
                           n_groups: int = 1, topk_groups: int = 1,
                           norm_topk: bool = False,
                           routed_scale: float = 1.0) -> np.ndarray:
    """Token-by-token evaluation with plain loops and full sorts (tiny inputs
    only).  Written independently of the vectorised path above."""
    import math
    x = np.asarray(x, np.float64)
    wg = np.asarray(w_gate, np.float64)
    T, d = x.shape
    E = wg.shape[0]
    f32 = np.float32
    routed_fn = _as_expert_fn(routed)
    shared_fn = _as_expert_fn(shared)
    y = np.zeros((T, d))
    for t in range(T):
        logits = []
        for e in range(E):
            acc = 0.0
            for j in range(d):
                acc += x[t, j] * wg[e, j]
            v = f32(acc)
            if logit_bias is not None:
                v = f32(v + f32(logit_bias[e]))
            logits.append(float(v))
        if score == "softmax":
            m = max(logits)
            ex = [math.exp(v - m) for v in logits]
            tot = math.fsum(ex)
            s = [float(f32(v / tot)) for v in ex]
        else:
            s = [float(f32(1.0 / (1.0 + math.exp(-v)))) for v in logits]
        key = [float(f32(s[e]) + (f32(select_bias[e]) if select_bias is not None
                                  else f32(0.0))) for e in range(E)]
        eligible = list(range(E))
        if n_groups > 1:
            gs = E // n_groups
            gscore = []
            for gi in range(n_groups):
                ks = sorted((key[e] for e in range(gi * gs, (gi + 1) * gs)),
                            reverse=True)
                gscore.append(float(f32(ks[0]) + f32(ks[1])) if gs > 1 else ks[0])
            best = sorted(range(n_groups), key=lambda gi: (-gscore[gi], gi))
            keep = set(best[:topk_groups])
            eligible = [e for e in range(E) if e // gs in keep]
        ranked = sorted(eligible, key=lambda e: (-key[e], e))
        sel = ranked[:top_k]
        g = [s[e] for e in sel]
        if norm_topk:
            tot = math.fsum(g)
            g = [v / tot for v in g]
        g = [v * routed_scale for v in g]
        u = x[t]
        out = u.copy()

        def ffn(w1, w3, w2):
            w1 = np.asarray(w1, np.float64)
            w3 = np.asarray(w3, np.float64)
            w2 = np.asarray(w2, np.float64)
            h = np.empty(w1.shape[0])
            for i in range(w1.shape[0]):
                a = float(np.dot(w1[i], u))
                b = float(np.dot(w3[i], u))
                h[i] = a / (1.0 + math.exp(-a)) * b
            return np.array([float(np.dot(w2[j], h)) for j in range(d)])
        for s_i in range(n_shared):
            out = out + ffn(*shared_fn(s_i))
        for k, e in enumerate(sel):
            out = out + g[k] * ffn(*routed_fn(e))
        y[t] = out
    return y


# ---------------------------------------------------------------------------
# Dispatch bookkeeping
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Dispatch:
    counts: np.ndarray     # [E] int64 tokens per routed expert
    offsets: np.ndarray    # [E+1] exclusive prefix sum of counts
    row_src: np.ndarray    # [T*K] token of each expert-contiguous row
    slot_row: np.ndarray   # [T, K] row holding token t's k-th kept expert


def dispatch(idx: np.ndarray, n_experts: int) -> Dispatch:
    """Expert-contiguous permutation of the (token, slot) pairs.

    Rows are ordered by (expert ascending, token ascending); every pair
    appears exactly once (nothing is dropped)."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    counts = np.bincount(idx.ravel(), minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    flat_e = idx.ravel()
    flat_t = np.repeat(np.arange(T), K)
    order = np.lexsort((flat_t, flat_e))          # by expert, then token
    row_src = flat_t[order]
    slot_row = np.empty(T * K, np.int64)
    slot_row[order] = np.arange(T * K)
    return Dispatch(counts=counts, offsets=offsets, row_src=row_src,
                    slot_row=slot_row.reshape(T, K))


# ---------------------------------------------------------------------------
# Work accounting
# ---------------------------------------------------------------------------

def activated_macs_per_token(d: int, n_routed: int, top_k: int, inner: int,
                             n_shared: int, shared_inner: int) -> int:
    """Multiply-adds per token: the gate (d per routed expert) plus three
    d x inner matrices for each of the K kept routed and K_s shared
    experts."""
    return d * n_routed + 3 * d * (top_k * inner + n_shared * shared_inner)


def expert_flops_per_token(d: int, top_k: int, inner: int, n_shared: int,
                           shared_inner: int) -> int:
    """FLOPs of the activated expert FFNs per token (2 per multiply-add)."""
    return 2 * 3 * d * (top_k * inner + n_shared * shared_inner)


def bias_update(counts, bias, gamma: float):
    """Auxiliary-loss-free load balancing, the step after a training forward
    pass (DeepSeek-V3 Technical Report summary, "2. Architecture": the
    per-expert bias is updated after each step by whether the expert was
    overloaded or underloaded).

    Reading of that sentence: with ``total`` tokens routed over ``n`` experts
    the balanced load is ``total / n``; an expert above it is overloaded and
    its bias goes down by ``gamma``, one below it is underloaded and its bias
    goes up by ``gamma``, one exactly at it keeps its bias.  The comparison
    ``count * n`` vs ``total`` is made on Python integers (exact); each update
    is a single fp32 addition.  Also returns the relative load
    ``count * n / total`` (1 = balanced), the exact quotient rounded to fp32.
    """
    counts = [int(c) for c in counts]
    n = len(counts)
    total = sum(counts)
    new = np.array(bias, dtype=np.float32).copy()
    g = np.float32(gamma)
    rel = np.zeros(n, dtype=np.float32)
    for e, c in enumerate(counts):
        if c * n > total:
            new[e] = np.float32(new[e] - g)
        elif c * n < total:
            new[e] = np.float32(new[e] + g)
        rel[e] = np.float32(c * n / total) if total > 0 else np.float32(0.0)
    return new, rel
