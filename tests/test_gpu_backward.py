"""GPU parity of the layer backward (moe_layer_backward through the C ABI)
against the backward oracle, on the same seeded inputs and the GPU's expert
choice.

Bar: every gradient element within 2e-2 * rms(reference tensor) (the bf16
layer's bound, which covers dx's own rounding at the output) plus, for the
results of products that take an operand rounded to bf16 -- the SwiGLU input
gradients dA (dW1, dW3 and dx's expert part) and g h (dW2) -- 2^-7 times the
sum of the absolute values of that product's terms (the oracle reports these
sums).  bf16 keeps 8 significant bits (relative rounding error <= 2^-9): dA
is rounded once, and each routed row's share of dx (and the shared experts'
share) once more before the shares are summed, so every term of dx moves by at
most about 2^-8 of its size and every term of a weight gradient by 2^-9;
2^-7 leaves room for the fp32 accumulation and the recomputed
pre-activations.  The expert choice must
equal the oracle's on every token whose selection margin exceeds 1e-5 and
equal the forward's on every token.

Sizes: reduced T with the full 16B hidden/inner/expert shapes (several N
tiles, ragged tails of rows per expert), a few experts with ~1000 rows each
(several M tiles and a long k loop in the weight gradients), the V3 routing
(sigmoid, groups, selection bias, renormalised) at d = 512, the skewed small
batch with a logit bias, no shared expert with every expert kept, a routed
scale, T = 0, bitwise reproducibility, and the full 16B-shaped layer on every
token and every weight gradient.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import MARGIN, Case

pytestmark = pytest.mark.gpu
TOL = 2e-2
C = workloads.CONFIGS
B16 = C["deepseekmoe-16b"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_backward(case, dout):
    import mixture_experts_layer_mk_amd as moe
    c, d = case.cfg, case.dev
    return moe.moe_layer_backward(
        d["x"], d["w_gate"], d["routed"], d["shared"], c.top_k, dout,
        score=c.score, norm_topk=c.norm_topk, n_groups=c.n_groups,
        topk_groups=c.topk_groups, select_bias=d["select_bias"],
        logit_bias=d["logit_bias"], routed_scale=c.routed_scale)


ROUND = 2.0 ** -7     # per unit of sum |terms| of a product with one bf16-rounded factor


def _close(name, got, ref, info, mag=None):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite"
    if not ref.size:
        return
    rms = np.sqrt(np.mean(ref ** 2))
    diff = np.abs(got - ref)
    info[name] = float(diff.max() / rms) if rms > 0 else float(diff.max())
    if mag is not None:
        diff = diff - ROUND * mag
    err = diff.max()
    assert err <= TOL * rms + 1e-30, f"{name}: max|err| {err:.3e} > {TOL} * rms {rms:.3e}"


def check_backward(case):
    cfg = case.cfg
    dout_np = workloads.make_inputs(cfg).dout()
    dout = torch.from_numpy(dout_np).to(torch.bfloat16).cuda()
    gr = run_backward(case, dout)
    torch.cuda.synchronize()
    idx = gr["topk_idx"].cpu().numpy()
    # the expert choice: the forward's on every token, the oracle's where clear
    import mixture_experts_layer_mk_amd as moe
    _, rt = moe.moe_layer_forward(
        case.dev["x"], case.dev["w_gate"], case.dev["routed"], case.dev["shared"],
        cfg.top_k, score=cfg.score, norm_topk=cfg.norm_topk, n_groups=cfg.n_groups,
        topk_groups=cfg.topk_groups, select_bias=case.dev["select_bias"],
        logit_bias=case.dev["logit_bias"], routed_scale=cfg.routed_scale,
        return_routing=True)
    assert np.array_equal(idx, rt["topk_idx"].cpu().numpy()), "choice differs from the forward's"
    kw = case.oracle_kw()
    r = oracle.route(case.x, case.w_gate, cfg.top_k, score=cfg.score,
                     logit_bias=case.logit_bias, select_bias=case.select_bias,
                     n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                     norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale)
    amb = (r.margin <= MARGIN) | (r.group_margin <= MARGIN)
    same = (np.sort(idx, 1) == np.sort(r.idx, 1)).all(1)
    assert (same | amb).all(), "choice differs from the oracle's on a clear token"

    host = lambda ws: tuple(w.float().numpy() for w in ws) if ws is not None else None
    ref = oracle.moe_backward(case.x, case.w_gate, host(case.host["routed"]),
                              host(case.host["shared"]), cfg.top_k, dout_np,
                              forced_idx=idx, magnitudes=True, **kw)
    info = {}
    _close("dx", gr["dx"].float().cpu().numpy(), ref.dx, info, ref.dx_mag)
    _close("dw_gate", gr["dw_gate"].cpu().numpy(), ref.dw_gate, info)
    if case.logit_bias is not None:
        _close("dlogit_bias", gr["dlogit_bias"].cpu().numpy(), ref.dlogit_bias, info)
    names = ("dw1", "dw3", "dw2")
    for j in range(3):
        _close("routed." + names[j], gr["routed"][j].cpu().numpy(), ref.routed[j], info,
               ref.routed_mag[j])
        if cfg.n_shared:
            _close("shared." + names[j], gr["shared"][j].cpu().numpy(), ref.shared[j], info,
                   ref.shared_mag[j])
    info["ambiguous"] = int(amb.sum())
    return info, gr


CASES = {
    "16b-small-d256": B16.replace(T=300, d=256, inner=128, shared_inner=128),
    "16b-T600": B16.replace(T=600, seed=1),
    "few-experts-long-k": B16.replace(T=2000, d=512, n_routed=4, top_k=2, inner=256,
                                      n_shared=1, shared_inner=384, seed=2),
    "v3-d512": C["deepseek-v3"].replace(T=256, d=512, inner=256, shared_inner=256, seed=3),
    "skewed-logit-bias": C["skewed-16b-small"],
    "no-shared-all-kept": B16.replace(T=333, d=256, n_routed=8, top_k=8, inner=128,
                                      n_shared=0, seed=4),
    "routed-scale": B16.replace(T=200, d=256, inner=192, shared_inner=64, routed_scale=2.5,
                                seed=5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    cfg = CASES[name]
    say(f"[bwd] {name}: {cfg}")
    info, _ = check_backward(Case(cfg))
    say(f"[bwd] {name}: {info}")


def test_backward_bitwise_reproducible():
    case = Case(B16.replace(T=257, d=256, inner=128, shared_inner=128, seed=6))
    dout = torch.from_numpy(workloads.make_inputs(case.cfg).dout()).to(torch.bfloat16).cuda()
    a = run_backward(case, dout)
    b = run_backward(case, dout)
    torch.cuda.synchronize()
    assert torch.equal(a["dx"], b["dx"]) and torch.equal(a["dw_gate"], b["dw_gate"])
    for j in range(3):
        assert torch.equal(a["routed"][j], b["routed"][j])
        assert torch.equal(a["shared"][j], b["shared"][j])


def test_backward_side_stream_matches_in_order():
    """Untraced backward calls run the shared experts' branch on a side stream
    (joined before the dx combine and at the end); a traced call runs every
    stage in order.  Every gradient is bitwise equal, on a repeated call too."""
    import mixture_experts_layer_mk_amd as moe
    case = Case(B16.replace(T=600, seed=8))
    c, d = case.cfg, case.dev
    dout = torch.from_numpy(workloads.make_inputs(c).dout()).to(torch.bfloat16).cuda()
    ev = moe.HipEvents(len(moe.backward_stage_names()) + 1)

    def run(events=None):
        return moe.moe_layer_backward(
            d["x"], d["w_gate"], d["routed"], d["shared"], c.top_k, dout,
            score=c.score, norm_topk=c.norm_topk, n_groups=c.n_groups,
            topk_groups=c.topk_groups, select_bias=d["select_bias"],
            logit_bias=d["logit_bias"], routed_scale=c.routed_scale, trace_events=events)
    try:
        ref = run(ev.handles)
        outs = [run(), run()]
        torch.cuda.synchronize()
    finally:
        ev.close()
    for o in outs:
        assert torch.equal(o["dx"], ref["dx"]) and torch.equal(o["dw_gate"], ref["dw_gate"])
        for j in range(3):
            assert torch.equal(o["routed"][j], ref["routed"][j])
            assert torch.equal(o["shared"][j], ref["shared"][j])


def test_backward_no_tokens_gives_zero_weight_gradients():
    import mixture_experts_layer_mk_amd as moe
    case = Case(B16.replace(T=64, d=256, inner=128, shared_inner=128, seed=7))
    d = case.dev
    x0 = d["x"][:0]
    gr = moe.moe_layer_backward(x0, d["w_gate"], d["routed"], d["shared"], 6, x0.clone())
    torch.cuda.synchronize()
    assert gr["dx"].numel() == 0
    assert not gr["dw_gate"].any()
    for t in gr["routed"] + gr["shared"]:
        assert not t.any()


def test_backward_full_size_all_tokens():
    """The full 16B-shaped layer (T = 16384, the shapes the benchmark times):
    dx of every token, every routed expert's weight gradients over all its
    rows, every shared expert's over all tokens, and the gate gradients,
    against the oracle run expert by expert."""
    say("[bwd-full] generating")
    case = Case(B16)
    say("[bwd-full] running")
    info, _ = check_backward(case)
    say(f"[bwd-full] {info}")
