"""GPU parity over a seeded sweep of layer shapes that the named workloads do
not reach: hidden sizes that are not a multiple of the 256-wide output tile,
inner sizes with a half tile, odd expert counts, K up to E, zero to two
shared experts, token counts from 1 to a few hundred; the forward in bf16,
fp32 and FP8 and the backward, each against the oracle with the same bars as
the workload tests."""
import sys

import numpy as np
import pytest
import torch

import workloads
from parity import Case, check_case
from test_gpu_backward import check_backward

pytestmark = pytest.mark.gpu
B16 = workloads.CONFIGS["deepseekmoe-16b"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _shape(seed, step=64):
    """A random layer shape (seeded); sizes multiples of `step`."""
    r = np.random.default_rng(1000 + seed)
    E = int(r.choice([1, 3, 9, 17, 40, 63]))
    K = int(r.integers(1, min(E, 8) + 1))
    Ks = int(r.integers(0, 3))
    mult = lambda lo, hi: int(r.integers(lo, hi + 1)) * step
    d = mult(2, 7)
    inner = mult(1, 6)
    sinner = mult(1, 4)
    T = int(r.choice([1, 37, 130, 300]))
    score = "sigmoid" if r.random() < 0.3 else "softmax"
    return B16.replace(T=T, d=d, n_routed=E, top_k=K, inner=inner, n_shared=Ks,
                       shared_inner=sinner, score=score, norm_topk=score == "sigmoid",
                       seed=seed)


@pytest.mark.parametrize("seed", range(8))
def test_forward_shapes_bf16(seed):
    cfg = _shape(seed)
    say(f"[shape bf16] {cfg}")
    say(f"[shape bf16] {check_case(Case(cfg))}")


@pytest.mark.parametrize("seed", range(4))
def test_forward_shapes_f32(seed):
    cfg = _shape(seed + 8).replace(dtype="f32")
    say(f"[shape f32] {cfg}")
    say(f"[shape f32] {check_case(Case(cfg))}")


@pytest.mark.parametrize("seed", range(4))
def test_forward_shapes_fp8(seed):
    cfg = _shape(seed + 12, step=128).replace(dtype="fp8")
    say(f"[shape fp8] {cfg}")
    say(f"[shape fp8] {check_case(Case(cfg))}")


@pytest.mark.parametrize("seed", range(6))
def test_backward_shapes(seed):
    cfg = _shape(seed + 16)
    say(f"[shape bwd] {cfg}")
    info, _ = check_backward(Case(cfg))
    say(f"[shape bwd] {info}")
