"""The seeded generator: reproducible, lazy access equals the full tensors,
bf16 workloads hold exactly representable values, and the draws have the
stated scales."""
import numpy as np
import pytest
import torch

import workloads


def test_reproducible_and_lazy_equals_full():
    a = workloads.make_inputs("tiny-fp32")
    b = workloads.make_inputs("tiny-fp32")
    np.testing.assert_array_equal(a.x(), b.x())
    np.testing.assert_array_equal(a.x_rows([5, 63, 0]), a.x()[[5, 63, 0]])
    full = a.torch_tensors()
    np.testing.assert_array_equal(full["x"].numpy(), a.x())
    np.testing.assert_array_equal(full["routed"][2][7].numpy(), a.routed(7)[2])
    np.testing.assert_array_equal(full["shared"][0][0].numpy(), a.shared(0)[0])
    assert not np.array_equal(a.x(), workloads.make_inputs("tiny-fp32", seed=1).x())


def test_bf16_values_are_exact():
    cfg = workloads.CONFIGS["deepseekmoe-16b"].replace(T=300, d=64, inner=32,
                                                       shared_inner=32, n_routed=8)
    inp = workloads.make_inputs(cfg)
    x = inp.x()
    assert np.array_equal(torch.from_numpy(x).bfloat16().float().numpy(), x)
    w1 = inp.routed(3)[0]
    assert np.array_equal(torch.from_numpy(w1).bfloat16().float().numpy(), w1)
    t = inp.torch_tensors()
    assert t["x"].dtype == torch.bfloat16 and t["w_gate"].dtype == torch.float32
    np.testing.assert_array_equal(t["x"].float().numpy(), x)


def test_scales_and_biases():
    cfg = workloads.CONFIGS["deepseekmoe-16b"].replace(T=2048, d=256, inner=128,
                                                       shared_inner=128, n_routed=8)
    inp = workloads.make_inputs(cfg)
    assert abs(inp.x().std() - 1) < 0.02
    assert abs(inp.w_gate().std() * np.sqrt(256) - 1) < 0.05
    w1, w3, w2 = inp.routed(0)
    assert abs(w1.std() * np.sqrt(256) - 1) < 0.05
    assert abs(w2.std() * np.sqrt(128) - 1) < 0.05
    v3 = workloads.make_inputs("deepseek-v3")
    sb = v3.select_bias()
    assert sb.shape == (256,) and np.abs(sb).max() <= 0.1 and v3.logit_bias() is None
    sk = workloads.make_inputs("skewed-16b-small")
    lb = sk.logit_bias()
    # a permutation of -1.2 ln r, r = 1..64
    np.testing.assert_allclose(np.sort(lb), np.sort(-1.2 * np.log(np.arange(1, 65))),
                               rtol=1e-6)
