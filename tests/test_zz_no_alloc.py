"""GPU test of the no-allocation forward (moe_layer_forward_noalloc): the
library's fixed per-device workspace instead of a caller's buffer.

Two calls in a row -- a 700-token 16B-shaped layer, then the 128-token skewed
batch (smaller) -- and a third, the tiny fp32 layer, each compared bitwise
with the allocating entry point (moe_layer_forward) on the same inputs: the
output, the kept experts, their weights and the per-expert counts.  The
buffer keeps the previous call's contents, so a stage that read stale
workspace would show here.  A layer too large for the buffer is refused with
MOE_ERR_SCRATCH before anything runs.
"""
import sys

import pytest
import torch

import workloads
from parity import Case

pytestmark = pytest.mark.gpu
C = workloads.CONFIGS


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(case, noalloc):
    import mixture_experts_layer_mk_amd as moe
    c, d = case.cfg, case.dev
    fn = moe.moe_layer_forward_noalloc if noalloc else moe.moe_layer_forward
    out = torch.full_like(d["x"], float("nan"))
    _, routing = fn(d["x"], d["w_gate"], d["routed"], d["shared"], c.top_k,
                    score=c.score, norm_topk=c.norm_topk, n_groups=c.n_groups,
                    topk_groups=c.topk_groups, select_bias=d["select_bias"],
                    logit_bias=d["logit_bias"], routed_scale=c.routed_scale,
                    out=out, return_routing=True)
    torch.cuda.synchronize()
    return out, routing


def test_noalloc_matches_allocating_forward():
    cases = [("16b-T700", C["deepseekmoe-16b"].replace(T=700, seed=12)),
             ("skewed-16b-small", C["skewed-16b-small"]),
             ("tiny-fp32", C["tiny-fp32"].replace(seed=5))]
    for name, cfg in cases:
        say(f"[noalloc] {name}: {cfg}")
        case = Case(cfg)
        ref, rref = _run(case, noalloc=False)
        out, rout = _run(case, noalloc=True)
        assert torch.equal(out, ref), f"{name}: output differs"
        for k in ("topk_idx", "topk_w", "expert_counts"):
            assert torch.equal(rout[k], rref[k]), f"{name}: {k} differs"
        say(f"[noalloc] {name}: bitwise equal")


def test_noalloc_rejects_oversize_layer():
    import mixture_experts_layer_mk_amd as moe
    cfg = C["deepseekmoe-16b"].replace(T=64, seed=13)
    case = Case(cfg)
    d = case.dev
    x = torch.zeros((4096, cfg.d), dtype=torch.bfloat16, device="cuda")
    desc = moe.make_desc(4096, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner, cfg.n_shared,
                         cfg.shared_inner)
    assert moe.workspace_size(desc) > moe.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(x, 7.0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(x, d["w_gate"], d["routed"], d["shared"], cfg.top_k,
                                      out=out)
    assert ei.value.status == moe.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "a refused call wrote its output"
