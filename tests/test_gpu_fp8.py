"""GPU parity of the FP8 layer (E4M3 expert GEMMs with power-of-two scales)
against the oracle of the FP8 layer, and of the quantisers against the
oracle's, bitwise.

Sizes: the FP8 workloads at reduced T with full hidden/inner/expert shapes
(several tiles, ragged tails), the full 16B-shaped layer on every token in
the launch configuration the benchmark times, and the edge cases (no shared
expert, the dense reduction, a weight block of zeros, large and tiny scales).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
import workloads
from parity import Case, check_case

pytestmark = pytest.mark.gpu

C = workloads.CONFIGS
F8 = C["deepseekmoe-16b-fp8"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_weight_quantiser_bitwise():
    import mixture_experts_layer_mk_amd as moe
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3, 256, 384)).astype(np.float32)
    w[0, :128, :128] = 0.0                                  # a block of zeros
    w[1, 128:, 256:] *= 2.0 ** 40                           # large scale
    w[2, :128, 128:256] *= 2.0 ** -60                       # tiny scale
    w[2, 5, 7] = -3e-20
    for dt in (torch.float32, torch.bfloat16):
        t = torch.from_numpy(w).to(dt)
        codes, scales = moe.quantize_fp8_blocks(t.cuda())
        torch.cuda.synchronize()
        host = t.float().numpy()
        for b in range(3):
            oc, os_ = ofp8.quantize_blocks(host[b])
            assert np.array_equal(codes[b].cpu().numpy(), oc), (dt, b)
            assert np.array_equal(scales[b].cpu().numpy(), os_), (dt, b)


REDUCED = {
    "16b-fp8-T2600": F8.replace(T=2600),
    "16b-fp8-T1000": F8.replace(T=1000, seed=1),
    "2b-fp8-T2000": C["deepseekmoe-2b"].replace(T=2000, dtype="fp8"),
    "v3-fp8-d512-T700": C["deepseek-v3"].replace(T=700, d=512, inner=256, shared_inner=256,
                                                  seed=2, dtype="fp8"),
    "skewed-fp8": C["skewed-16b-small"].replace(dtype="fp8"),
    # group-limited routing with 2048 tokens: the split router and the token
    # rows quantised on the side stream
    "v3-fp8-d512-T2048": C["deepseek-v3"].replace(T=2048, d=512, inner=256, shared_inner=256,
                                                  dtype="fp8", seed=11),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_fp8_reduced_all_tokens(name):
    cfg = REDUCED[name]
    say(f"[fp8] {name}: {cfg}")
    info = check_case(Case(cfg))
    say(f"[fp8] {name}: {info}")


def test_fp8_intermediates_against_oracle():
    """The E4M3 token rows and their scales read back from the workspace equal
    the oracle's bitwise, and every SwiGLU activation code (routed rows and
    shared experts) is admissible under the accumulation bound (both inside
    check_case); the share of codes that are not the nearest to the exact H
    is reported."""
    cfg = F8.replace(T=777, seed=3)
    info = check_case(Case(cfg))
    assert info["h_codes"] == cfg.T * (cfg.top_k * cfg.inner + cfg.n_shared * cfg.shared_inner)
    say(f"[fp8] H: {info['h_codes_not_nearest']} of {info['h_codes']} codes are not the "
        f"nearest to the exact activation; {info}")


@pytest.mark.parametrize("Ks", [0, 1])
def test_fp8_no_shared_and_dense(Ks):
    if Ks == 0:
        cfg = F8.replace(T=333, n_routed=8, top_k=8, n_shared=0, d=256, inner=128)
    else:
        cfg = F8.replace(T=500, n_routed=1, top_k=1, n_shared=0, d=512, inner=384)
    info = check_case(Case(cfg))
    say(f"[fp8] Ks={Ks}: {info}")


def test_fp8_full_size_all_tokens():
    """The full 16B-shaped FP8 layer in the launch configuration the benchmark
    times, every token, every activation code."""
    say("[fp8-full] generating")
    case = Case(F8)
    say("[fp8-full] running")
    info = check_case(case)
    say(f"[fp8-full] {info}")


def test_fp8_error_against_bf16_layer():
    """What FP8 costs: the FP8 layer against the bf16-exact oracle of the same
    layer (informational bound: quantisation-sized, a few percent of the
    expert contribution)."""
    cfg = F8.replace(T=512, seed=9)
    case = Case(cfg)
    out, routing = case.run_gpu()
    torch.cuda.synchronize()
    rows = np.arange(cfg.T)
    idx = routing["topk_idx"].cpu().numpy()
    y, _ = oracle.moe_forward(case.x, case.w_gate, case.routed, case.shared, cfg.top_k,
                              forced_idx=idx, **case.oracle_kw())
    g = out.float().cpu().numpy()
    rel = np.sqrt(np.mean((g - y) ** 2)) / np.sqrt(np.mean((y - case.x) ** 2))
    say(f"[fp8] rms error vs bf16-exact layer, relative to the expert contribution: {rel:.4f}")
    assert rel < 0.1
