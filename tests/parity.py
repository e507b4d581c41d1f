"""Shared logic of the GPU parity tests: run the HIP layer and the CPU oracle
on the same seeded inputs and compare them under the stated rules.

Rules (the layer's acceptance criteria):
* routing: for every token whose K-th and (K+1)-th selection keys (and, with
  group-limited routing, whose kept and first dropped group scores) differ by
  more than 1e-5, the kept experts must be exactly the oracle's.  Tokens
  inside that margin may take any choice that is optimal within 1e-5; the
  GPU's choice is checked for that and the output is compared with the oracle
  run on the GPU's choice.
* per-expert counts equal the histogram of the GPU's choices (exactly), and
  equal the oracle's when no token is ambiguous.
* outputs: max |err| <= 2e-2 * rms(out) for bf16 layers, <= 1e-4 * rms(out)
  for fp32 layers, against the fp64 oracle.
* FP8 layers: the E4M3 SwiGLU activations H the GPU quantised (read back
  from the workspace, with their 1x128 scales) must each be admissible: the
  quantisation of some value of h = silu(a1) a3 reachable when each gate/up
  pre-activation a = sum_j t_j is off by at most ``FP8_ACC_REL`` * sum_j |t_j|
  (the accumulation bound the layer is held to; fixed, not measured).  Where
  H admits several codes the GPU's is one correct choice, so the output is
  then compared, at the bf16 bar 2e-2 * rms(out) and with no further
  allowance, with the oracle of the FP8 layer evaluated on those codes (the
  same E4M3 token rows, weights and routing; exact accumulation of the
  down-projections).  The raw error against the oracle's own exact-H layer is
  reported beside.  The weights' codes and scales (from the library's
  quantiser) and the token rows' must equal the oracle's bitwise.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import oracle.fp8
import workloads
from mixture_experts_layer_mk_amd import moe_layer_forward, quantize_fp8_blocks

MARGIN = 1e-5
_ORACLE_Q = {}   # the oracle's E4M3 weights, per (part, seed, shapes)
# Accumulation bound of the FP8 layer's gate/up products: each pre-activation
# may be off by at most this fraction of the sum of its terms' magnitudes.
# The pages say only that FP8 accumulation is limited and must be made
# precise; 2^-10 (a 10-bit significand applied once to the whole sum) is the
# reading fixed here, finer than the layer's own bf16 activations (8 bits).
FP8_ACC_REL = 2.0 ** -10
TOL = {"bf16": 2e-2, "f32": 1e-4, "fp8": 2e-2}


class Case:
    """One workload: host tensors (generator output), device copies, and the
    oracle's view of the same values."""

    def __init__(self, cfg: workloads.LayerConfig, seed: int = 0, device="cuda"):
        self.cfg = cfg
        self.inp = workloads.make_inputs(cfg, seed)
        self.host = self.inp.torch_tensors(
            "cpu", progress=lambda m: print(f"[{cfg.name}] {m}", flush=True))
        self.dev = {k: (tuple(t.to(device) for t in v) if isinstance(v, tuple)
                        else (v.to(device) if v is not None else None))
                    for k, v in self.host.items()}
        h = self.host
        self.x = h["x"].float().numpy()
        self.w_gate = h["w_gate"].numpy()
        self.logit_bias = None if h["logit_bias"] is None else h["logit_bias"].numpy()
        self.select_bias = None if h["select_bias"] is None else h["select_bias"].numpy()
        if cfg.dtype == "fp8":
            self._quantize_fp8()

    def _quantize_fp8(self):
        """Weights to E4M3 + block scales with the library's quantiser (device
        copies) and with the oracle's (host); the two must agree bitwise."""
        self.dev_q, self.dev_s, self.ora_q = {}, {}, {}
        for key in ("routed", "shared"):
            ws = self.dev[key]
            if ws is None:
                self.dev_q[key] = self.dev_s[key] = self.ora_q[key] = None
                continue
            q = [quantize_fp8_blocks(w) for w in ws]
            torch.cuda.synchronize()
            self.dev_q[key] = tuple(c for c, _ in q)
            self.dev_s[key] = tuple(s for _, s in q)
            # the weights depend on the seed and the expert shapes only
            c = self.cfg
            ck = (key, self.inp.seed, c.d, c.n_routed, c.inner, c.n_shared, c.shared_inner)
            if ck not in _ORACLE_Q:
                host = [w.float().numpy() for w in self.host[key]]
                _ORACLE_Q[ck] = oracle.fp8.quantize_experts(*host)
            self.ora_q[key] = _ORACLE_Q[ck]
            for (c, s), (oc, os_) in zip(q, self.ora_q[key]):
                assert np.array_equal(c.cpu().numpy(), oc), f"{key}: codes differ"
                assert np.array_equal(s.cpu().numpy(), os_), f"{key}: scales differ"

    def routed(self, e):
        w1, w3, w2 = self.host["routed"]
        return (w1[e].float().numpy(), w3[e].float().numpy(), w2[e].float().numpy())

    def shared(self, s):
        w1, w3, w2 = self.host["shared"]
        return (w1[s].float().numpy(), w3[s].float().numpy(), w2[s].float().numpy())

    def run_gpu(self, **kw):
        c, d = self.cfg, self.dev
        if c.dtype == "fp8":
            kw = dict(kw, expert_scales=self.dev_s["routed"],
                      shared_scales=self.dev_s["shared"])
            routed, shared = self.dev_q["routed"], self.dev_q["shared"]
        else:
            routed, shared = d["routed"], d["shared"]
        return moe_layer_forward(
            d["x"], d["w_gate"], routed, shared, c.top_k,
            score=c.score, norm_topk=c.norm_topk, n_groups=c.n_groups,
            topk_groups=c.topk_groups, select_bias=d["select_bias"],
            logit_bias=d["logit_bias"], routed_scale=c.routed_scale,
            return_routing=True, **kw)

    def oracle_kw(self):
        c = self.cfg
        return dict(n_shared=c.n_shared, score=c.score, logit_bias=self.logit_bias,
                    select_bias=self.select_bias, n_groups=c.n_groups,
                    topk_groups=c.topk_groups, norm_topk=c.norm_topk,
                    routed_scale=c.routed_scale)

    def oracle(self, rows, forced_idx=None, forced_h=None):
        if self.cfg.dtype == "fp8":
            return oracle.fp8.moe_forward_fp8(
                self.x[rows], self.w_gate, self.ora_q["routed"], self.ora_q["shared"],
                self.cfg.top_k, forced_idx=forced_idx, forced_h=forced_h,
                **self.oracle_kw())
        return oracle.moe_forward(self.x[rows], self.w_gate, self.routed,
                                  self.shared if self.cfg.n_shared else None,
                                  self.cfg.top_k, forced_idx=forced_idx,
                                  **self.oracle_kw())


def choice_is_near_optimal(keys_unmasked, choice, cfg, tol=MARGIN) -> bool:
    """Is `choice` a top-K that is optimal up to `tol` (group limit included)?"""
    E, K = keys_unmasked.size, cfg.top_k
    key = keys_unmasked.astype(np.float64)
    if len(set(choice)) != K:
        return False
    if cfg.n_groups > 1:
        gs = E // cfg.n_groups
        G = np.array([np.sort(key[g * gs:(g + 1) * gs])[-2:].sum()
                      for g in range(cfg.n_groups)])
        chosen_groups = sorted({int(e) // gs for e in choice})
        if len(chosen_groups) > cfg.topk_groups:
            return False
        g_cut = np.sort(G)[::-1][cfg.topk_groups - 1]
        if any(G[g] < g_cut - tol for g in chosen_groups):
            return False
        # kept groups: the chosen ones plus the best of the rest
        rest = [g for g in np.argsort(-G, kind="stable") if g not in chosen_groups]
        kept = chosen_groups + rest[:cfg.topk_groups - len(chosen_groups)]
        eligible = [e for e in range(E) if e // gs in kept]
    else:
        eligible = list(range(E))
    unchosen = [e for e in eligible if e not in set(choice)]
    if not unchosen:
        return True
    return min(key[list(choice)]) >= max(key[unchosen]) - tol


def _workspace(cfg):
    from mixture_experts_layer_mk_amd import make_desc, workspace_layout, workspace_size
    desc = make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner, cfg.n_shared,
                     cfg.shared_inner, n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                     score=cfg.score, norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale,
                     dtype=cfg.dtype)
    ws = torch.empty(max(workspace_size(desc), 1), dtype=torch.uint8, device="cuda")
    return ws, workspace_layout(desc)


def fp8_admissible_h(case: Case, ws, lay, idx):
    """Check every E4M3 SwiGLU activation the GPU quantised (routed rows and
    shared experts, read back from the workspace) against the interval the
    accumulation bound allows; return the GPU's H as the oracle's forced_h
    (dequantised) and counts for the report."""
    from oracle import fp8
    cfg = case.cfg
    T, K, I = cfg.T, cfg.top_k, cfg.inner
    ws_np = ws.cpu().numpy()

    def view(off, n, dt):
        return ws_np[off:off + n * np.dtype(dt).itemsize].view(dt)
    slot_row = view(lay["slot_row_i32"], T * K, np.int32).reshape(T, K)
    xd = fp8.dequantize_1x128(*fp8.quantize_1x128(case.x))
    info = {"h_codes": 0, "h_codes_not_nearest": 0}

    def check(name, rows_x, w1q, w3q, codes, scales):
        W1, W3 = fp8.dequantize_blocks(*w1q), fp8.dequantize_blocks(*w3q)
        h, lo, hi = fp8.activation_interval(rows_x, W1, W3, FP8_ACC_REL)
        ok, _ = fp8.admissible_1x128(lo, hi, codes, scales)
        bad = np.argwhere(~ok)
        assert bad.size == 0, (f"{name}: {len(bad)} FP8 activations outside their "
                               f"admissible interval, e.g. {bad[0]}")
        own_c, own_s = fp8.quantize_1x128(h)
        info["h_codes"] += codes.size
        info["h_codes_not_nearest"] += int(
            (fp8.dequantize_1x128(own_c, own_s) != fp8.dequantize_1x128(codes, scales)).sum())
        return fp8.dequantize_1x128(codes, scales)

    (c1, s1), (c3, s3), _ = case.ora_q["routed"]
    hr = view(lay["h_routed"], T * K * I, np.uint8).reshape(T * K, I)
    hrs = view(lay["h_routed_scale"], T * K * (I // 128), np.uint8).reshape(T * K, I // 128)
    forced_r = np.zeros((T, K, I))
    for e in np.unique(idx):
        tt, kk = np.nonzero(idx == e)
        rows = slot_row[tt, kk]
        forced_r[tt, kk] = check(f"routed expert {e}", xd[tt], (c1[e], s1[e]),
                                 (c3[e], s3[e]), hr[rows], hrs[rows])
    forced_s = []
    if cfg.n_shared:
        Is = cfg.shared_inner
        ksi = cfg.n_shared * Is
        hs = view(lay["h_shared"], T * ksi, np.uint8).reshape(T, ksi)
        hss = view(lay["h_shared_scale"], T * ksi // 128, np.uint8).reshape(T, ksi // 128)
        (q1, t1), (q3, t3), _ = case.ora_q["shared"]
        for si in range(cfg.n_shared):
            cols = slice(si * Is, (si + 1) * Is)
            gcols = slice(si * Is // 128, (si + 1) * Is // 128)
            forced_s.append(check(f"shared expert {si}", xd, (q1[si], t1[si]),
                                  (q3[si], t3[si]), hs[:, cols], hss[:, gcols]))
    # the token rows the experts read: bitwise the oracle's quantisation
    xq = view(lay["x_q"], T * cfg.d, np.uint8).reshape(T, cfg.d)
    xs = view(lay["x_scale"], T * cfg.d // 128, np.uint8).reshape(T, cfg.d // 128)
    oc, os_ = fp8.quantize_1x128(case.x)
    assert np.array_equal(xq, oc) and np.array_equal(xs, os_), "token rows differ"
    return (forced_s, forced_r), info


def check_case(case: Case, rows=None, out=None, routing=None):
    """Run (unless given) the GPU layer, compare rows `rows` (default all)
    with the oracle; return a dict of diagnostics."""
    cfg = case.cfg
    fp8_layer = cfg.dtype == "fp8"
    ws = lay = None
    if fp8_layer:
        assert out is None and rows is None, "FP8 layers are checked on every token"
        ws, lay = _workspace(cfg)
        out, routing = case.run_gpu(workspace=ws)
    elif out is None:
        out, routing = case.run_gpu()
    torch.cuda.synchronize()
    T, K = cfg.T, cfg.top_k
    g_idx = routing["topk_idx"].cpu().numpy()
    g_w = routing["topk_w"].cpu().numpy()
    g_cnt = routing["expert_counts"].cpu().numpy()
    g_out = out.float().cpu().numpy()

    # properties at any size
    assert g_idx.min() >= 0 and g_idx.max() < cfg.n_routed
    assert (np.sort(g_idx, 1)[:, 1:] != np.sort(g_idx, 1)[:, :-1]).all(), "repeated expert"
    assert np.array_equal(g_cnt, np.bincount(g_idx.ravel(), minlength=cfg.n_routed))
    assert g_cnt.sum() == T * K
    assert np.isfinite(g_out).all()

    rows = np.arange(T) if rows is None else np.asarray(rows)
    r = oracle.route(case.x[rows], case.w_gate, K, score=cfg.score,
                     logit_bias=case.logit_bias, select_bias=case.select_bias,
                     n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                     norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale)
    amb = (r.margin <= MARGIN) | (r.group_margin <= MARGIN)
    gi = g_idx[rows]
    same = (np.sort(gi, 1) == np.sort(r.idx, 1)).all(1)
    bad = np.nonzero(~same & ~amb)[0]
    assert bad.size == 0, (f"routing differs on {bad.size} unambiguous tokens, "
                           f"e.g. row {rows[bad[0]]}: gpu {gi[bad[0]]} oracle {r.idx[bad[0]]}")
    unmasked = r.scores.astype(np.float32)
    if case.select_bias is not None:
        unmasked = unmasked + case.select_bias[None, :]
    for i in np.nonzero(amb & ~same)[0]:
        assert choice_is_near_optimal(unmasked[i], gi[i], cfg), f"row {rows[i]}"
    # order: keys non-increasing along k (within the tie tolerance)
    kk = np.take_along_axis(unmasked, gi.astype(np.int64), 1).astype(np.float64)
    assert (np.diff(kk, axis=1) <= MARGIN).all(), "kept experts not in key order"
    if amb.sum() == 0 and rows.size == T:
        ref_cnt = np.bincount(r.idx.ravel(), minlength=cfg.n_routed)
        assert np.array_equal(g_cnt, ref_cnt)

    # gate weights and outputs against the oracle run on the GPU's choice
    # (FP8: and on the GPU's admissible activation codes)
    info = {}
    forced_h = None
    if fp8_layer:
        forced_h, hinfo = fp8_admissible_h(case, ws, lay, gi)
        info.update(hinfo)
    y_ref, r_f = case.oracle(rows, forced_idx=gi, forced_h=forced_h)
    np.testing.assert_allclose(g_w[rows], r_f.g, rtol=1e-5, atol=1e-7)
    diff = np.abs(g_out[rows] - y_ref)
    rms = np.sqrt(np.mean(y_ref ** 2))
    tol = TOL[cfg.dtype]
    err = diff.max()
    if fp8_layer:
        y_exact, _ = case.oracle(rows, forced_idx=gi)
        info["max_err_over_rms_exact_h"] = float(np.abs(g_out[rows] - y_exact).max() / rms)
    assert err <= tol * rms, f"max|err| {err:.3e} > {tol} * rms {rms:.3e}"
    info.update({"err_over_rms": err / rms, "ambiguous": int(amb.sum()),
                 "rows": int(rows.size)})
    return info
