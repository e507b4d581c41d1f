"""Host-side pieces of bench.py (no GPU): it refuses more than one GPU
before touching any device, and the work it prices is the oracle's.

* The gate/up launch's FLOPs are two thirds of the layer's expert FLOPs (W1
  and W3 of every kept routed and every shared expert, against W2), and the
  expert FLOPs per token are pinned to the oracle's multiply-add counter in
  test_oracle_pins.
* The HBM bytes of a forward are the weights of the experts that receive a
  token plus the shared ones, x, the output and the fp32 gate.
"""
import os
import subprocess
import sys

import numpy as np

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gateup_flops_are_two_thirds_of_the_expert_flops():
    for name in ("deepseekmoe-16b", "deepseekmoe-2b", "deepseek-v3", "skewed-16b-small"):
        cfg = workloads.CONFIGS[name]
        per_token = oracle.expert_flops_per_token(cfg.d, cfg.top_k, cfg.inner, cfg.n_shared,
                                                  cfg.shared_inner)
        assert 3 * bench.gateup_flops(cfg) == 2 * cfg.T * per_token
    # the 16B-shaped launch: 1.512 TFLOP (routed 1.134 + shared 0.378)
    assert round(bench.gateup_flops(workloads.CONFIGS["deepseekmoe-16b"]) / 1e9) == 1512


def test_layer_hbm_bytes():
    cfg = workloads.CONFIGS["skewed-16b-small"]
    counts = np.zeros(cfg.n_routed, np.int64)
    counts[[0, 5, 9]] = [100, 1, 667]
    b, nonempty = bench.layer_hbm_bytes(cfg, counts)
    assert nonempty == 3
    weights = 2 * 3 * cfg.d * (3 * cfg.inner + cfg.n_shared * cfg.shared_inner)
    assert b == weights + 2 * 2 * cfg.T * cfg.d + 4 * cfg.n_routed * cfg.d
