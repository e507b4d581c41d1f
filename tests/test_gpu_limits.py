"""GPU parity at the boundary's limits, which the named workloads and the
shape sweep do not reach: the largest top-K (32) over the most routed
experts (256) with the group limit, 64 expert groups of one expert each, and
a top-K of 16 on a batch above a thousand tokens (past the fused router's
top-K of 8).  Forward in bf16 and fp32 and the backward, each against the
oracle with the same bars as the workload tests."""
import sys

import pytest
import torch

import workloads
from parity import Case, check_case
from test_gpu_backward import check_backward

pytestmark = pytest.mark.gpu
B16 = workloads.CONFIGS["deepseekmoe-16b"]
V3 = workloads.CONFIGS["deepseek-v3"]

CASES = {
    # 256 experts in 8 groups, 4 kept, 32 experts per token (the largest K)
    "v3-256-experts-top32": V3.replace(T=300, d=512, inner=128, shared_inner=128,
                                       top_k=32),
    # 64 groups of one expert: a group's score is its one key; 16 groups kept
    "64-groups-of-one": B16.replace(T=400, d=256, inner=128, shared_inner=128,
                                    n_groups=64, topk_groups=16, score="sigmoid",
                                    norm_topk=True),
    # top-16 on 1500 tokens: the split router with 64-token blocks
    "top16-1500-tokens": B16.replace(T=1500, d=256, inner=128, shared_inner=128,
                                     top_k=16),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(CASES))
def test_limits_forward_bf16(name):
    say(f"[limits bf16] {name}")
    say(f"[limits bf16] {check_case(Case(CASES[name]))}")


def test_limits_forward_f32():
    cfg = CASES["v3-256-experts-top32"].replace(dtype="f32")
    say("[limits f32] v3-256-experts-top32")
    say(f"[limits f32] {check_case(Case(cfg))}")


@pytest.mark.parametrize("name", ["v3-256-experts-top32", "top16-1500-tokens"])
def test_limits_backward(name):
    say(f"[limits bwd] {name}")
    info, _ = check_backward(Case(CASES[name]))
    say(f"[limits bwd] {info}")
