"""The every-token GPU parity tests at the full 16B and 2B shapes reach each
routed tail-tile layout of the 256-row GEMM launches.

An expert's last M-tile holds its remaining rows (the count modulo 256) and
runs the 64-, 128- or 192-row layout, the smallest that holds them, or the
full 256-row one.  This CPU test routes those workloads with the oracle and
checks that every layout occurs, so that a fault in any of them would show in
the GPU tests' comparisons.  It reads only the oracle's routing (the expert
counts), which the GPU path matches bit for bit under the margin rule.
"""
import numpy as np

import oracle
import workloads


def _tail_layouts(name):
    cfg = workloads.CONFIGS[name]
    h = workloads.make_inputs(cfg).torch_tensors("cpu")
    r = oracle.route(h["x"].float().numpy(), h["w_gate"].numpy(), cfg.top_k)
    counts = np.bincount(r.idx.ravel(), minlength=cfg.n_routed)
    # the launch's tile height: 256 when an expert averages at least 192 rows
    assert cfg.T * cfg.top_k // cfg.n_routed >= 192
    tails = counts % 256
    return {64 * int(np.ceil(t / 64)) for t in tails if t > 0} | (
        {256} if (counts >= 256).any() else set())


def test_full_size_routings_reach_every_tail_layout():
    seen = _tail_layouts("deepseekmoe-16b") | _tail_layouts("deepseekmoe-2b")
    assert seen == {64, 128, 192, 256}, seen
