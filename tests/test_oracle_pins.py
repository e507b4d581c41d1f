"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a closed form, a library
routine the oracle does not use, brute force, an invariant of the definition,
or a number printed on the pages (``tests/golden/page_numbers.json``).  The
tests are chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, T, d, E, I, Ks=0, Is=None):
    Is = I if Is is None else Is
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / math.sqrt(d)
    routed = (rng.standard_normal((E, I, d)) / math.sqrt(d),
              rng.standard_normal((E, I, d)) / math.sqrt(d),
              rng.standard_normal((E, d, I)) / math.sqrt(I))
    shared = None
    if Ks:
        shared = (rng.standard_normal((Ks, Is, d)) / math.sqrt(d),
                  rng.standard_normal((Ks, Is, d)) / math.sqrt(d),
                  rng.standard_normal((Ks, d, Is)) / math.sqrt(Is))
    return x, wg, routed, shared


# ---------------------------------------------------------------------------
# Expert FFN
# ---------------------------------------------------------------------------

def test_ffn_selection_matrices_closed_form():
    """W1, W3 pick coordinates p(i), q(i) of u; W2 scatters h_i to r(i).
    Then FFN(u)_j = sum_{i: r(i)=j} silu(u_p(i)) * u_q(i) with silu written
    with math.exp.  Non-square shapes catch transposed operands; distinct
    p and q catch swapped W1/W3."""
    rng = np.random.default_rng(1)
    d, I = 5, 7
    p = rng.integers(0, d, I)
    q = (p + 1 + rng.integers(0, d - 1, I)) % d
    r = rng.integers(0, d, I)
    w1 = np.zeros((I, d)); w1[np.arange(I), p] = 1
    w3 = np.zeros((I, d)); w3[np.arange(I), q] = 1
    w2 = np.zeros((d, I)); w2[r, np.arange(I)] = 1
    u = rng.standard_normal((3, d)) * 2
    got = oracle.swiglu_ffn(u, w1, w3, w2)
    want = np.zeros((3, d))
    for t in range(3):
        for i in range(I):
            a = u[t, p[i]]
            want[t, r[i]] += a / (1 + math.exp(-a)) * u[t, q[i]]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_ffn_matches_torch_textbook():
    """SwiGLU against torch.nn.functional (silu, linear) in fp64, a library
    path the oracle does not call."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(2)
    d, I = 24, 40
    u = rng.standard_normal((9, d))
    w1, w3 = rng.standard_normal((I, d)), rng.standard_normal((I, d))
    w2 = rng.standard_normal((d, I))
    T = lambda a: torch.from_numpy(a)
    want = F.linear(F.silu(F.linear(T(u), T(w1))) * F.linear(T(u), T(w3)), T(w2))
    np.testing.assert_allclose(oracle.swiglu_ffn(u, w1, w3, w2), want.numpy(),
                               rtol=1e-12, atol=1e-12)


def test_silu_special_values():
    """silu(0) = 0; silu(ln 3) = (3/4) ln 3; silu(a) - silu(-a) = a."""
    a = np.array([0.0, math.log(3.0), 2.5, -7.0])
    s = oracle.silu(a)
    assert s[0] == 0.0
    assert math.isclose(s[1], 0.75 * math.log(3.0), rel_tol=1e-15)
    np.testing.assert_allclose(s - oracle.silu(-a), a, atol=1e-14)


# ---------------------------------------------------------------------------
# Gate and selection
# ---------------------------------------------------------------------------

def test_gate_closed_forms():
    """d = 1, x = 1: logits are the gate entries.  softmax([ln 3, 0]) =
    (3/4, 1/4); sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2; a logit bias of
    -ln 3 cancels the first logit."""
    x = np.ones((1, 1))
    wg = np.array([[math.log(3.0)], [0.0]])
    s = oracle.gate_scores(oracle.gate_logits(x, wg), "softmax")
    np.testing.assert_allclose(s[0], [0.75, 0.25], rtol=1e-7)
    s = oracle.gate_scores(oracle.gate_logits(x, wg), "sigmoid")
    np.testing.assert_allclose(s[0], [0.75, 0.5], rtol=1e-7)
    l = oracle.gate_logits(x, wg, logit_bias=np.array([-math.log(3.0), 0.0]))
    assert abs(float(l[0, 0])) < 1e-7 and l[0, 1] == 0.0


def test_gate_logits_orientation():
    """l[t, e] = sum_j x[t, j] wg[e, j] with integer data (exact)."""
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, (4, 6)).astype(float)
    wg = rng.integers(-3, 4, (5, 6)).astype(float)
    l = oracle.gate_logits(x, wg)
    for t in range(4):
        for e in range(5):
            assert l[t, e] == sum(x[t, j] * wg[e, j] for j in range(6))


def test_topk_matches_full_stable_sort():
    """Top-K with many exact ties equals the first K of a full sort by
    (key descending, index ascending)."""
    rng = np.random.default_rng(4)
    s = (rng.integers(0, 5, (200, 12)) / 8.0).astype(np.float32)
    idx, _, margin, _ = oracle.select_experts(s, 5)
    for t in range(200):
        ref = sorted(range(12), key=lambda e: (-s[t, e], e))[:5]
        assert list(idx[t]) == ref
        assert margin[t] == float(s[t, ref[4]]) - float(
            s[t, sorted(range(12), key=lambda e: (-s[t, e], e))[5]])


def test_group_limit_is_optimal_exhaustive():
    """Group-limited top-K: the kept groups maximise the summed group score
    over every choice of groups, and the kept experts maximise the summed
    key over every K-subset of the eligible experts (enumerated)."""
    rng = np.random.default_rng(5)
    E, G, keep, K = 12, 4, 2, 4
    gs = E // G
    for _ in range(60):
        s = rng.random((1, E)).astype(np.float32)
        b = (rng.random(E) * 0.2 - 0.1).astype(np.float32)
        idx, keys, _, _ = oracle.select_experts(s, K, b, G, keep)
        key = (s[0] + b).astype(np.float64)
        gscore = [sum(sorted(key[g * gs:(g + 1) * gs])[-2:]) for g in range(G)]
        best_groups = max(itertools.combinations(range(G), keep),
                          key=lambda c: sum(gscore[g] for g in c))
        chosen_groups = sorted({int(e) // gs for e in idx[0]})
        assert set(chosen_groups) <= set(best_groups)
        eligible = [e for e in range(E) if e // gs in best_groups]
        best = max(itertools.combinations(eligible, K),
                   key=lambda c: sum(key[e] for e in c))
        assert sorted(idx[0]) == sorted(best)
        # masked keys are -inf exactly outside the kept groups
        for e in range(E):
            assert (keys[0, e] == -np.inf) == (e // gs not in best_groups)


def test_group_limit_ties_take_lowest_indices():
    """Equal group scores go to the lower group index and equal keys to the
    lower expert index (a total order on both).  Written-out cases:

    * every key equal (zero gate, sigmoid, no bias; 8 groups of 32, keep 4):
      groups 0..3 stay and experts 0..7 are kept, in index order;
    * groups 1 and 6 lead with equal scores, the other six tie below them:
      groups 1 and 6 stay, then 0 and 2; the four raised experts come first
      (index order), then the lowest-index experts of group 0."""
    T, d, E, K = 3, 16, 256, 8
    x = np.random.default_rng(21).standard_normal((T, d)).astype(np.float32)
    wg = np.zeros((E, d), np.float32)
    r = oracle.route(x, wg, K, score="sigmoid", n_groups=8, topk_groups=4, norm_topk=True)
    assert (r.idx == np.arange(8)[None, :]).all()
    assert np.all(r.g == 1.0 / 8)
    assert (r.margin == 0).all() and (r.group_margin == 0).all()
    bias = np.zeros(E, np.float32)
    raised = [32 + 5, 32 + 17, 192 + 3, 192 + 30]
    bias[raised] = np.float32(0.01)
    r = oracle.route(x, wg, K, score="sigmoid", select_bias=bias, n_groups=8,
                     topk_groups=4, norm_topk=True)
    assert (r.idx == np.array(raised + [0, 1, 2, 3])[None, :]).all()
    # the unbiased scores weigh the kept experts: all equal
    assert np.all(r.g == 1.0 / 8)
    ref = oracle.moe_forward_bruteforce(
        x, wg, lambda e: (np.eye(4, d, dtype=np.float32),) * 2 + (np.eye(d, 4, dtype=np.float32),),
        None, K, score="sigmoid", select_bias=bias, n_groups=8, topk_groups=4,
        norm_topk=True)
    y, _ = oracle.moe_forward(
        x, wg, lambda e: (np.eye(4, d, dtype=np.float32),) * 2 + (np.eye(d, 4, dtype=np.float32),),
        None, K, score="sigmoid", select_bias=bias, n_groups=8, topk_groups=4, norm_topk=True)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # softmax with groups: a zero gate makes every softmax score 1/E
    r = oracle.route(x, wg, 6, score="softmax", n_groups=4, topk_groups=2)
    assert (r.idx == np.arange(6)[None, :]).all()


def test_selection_bias_changes_choice_not_weight():
    """The selection bias steers the choice but the gate weight is the
    unbiased score: a large bias on expert 3 forces it in with weight s_3."""
    rng = np.random.default_rng(6)
    x, wg, routed, _ = rand_layer(rng, 8, 16, 6, 4)
    bias = np.zeros(6, np.float32); bias[3] = 10.0
    r = oracle.route(x, wg, 2, score="sigmoid", select_bias=bias)
    assert (r.idx[:, 0] == 3).all()
    np.testing.assert_array_equal(r.g[:, 0], r.scores[:, 3].astype(np.float64))


def test_gate_weight_sums():
    """Softmax scores sum to 1; the K kept softmax weights sum to at least
    K/E (the K largest of E numbers averaging 1/E) and at most 1, exactly 1
    when K = E; renormalised weights sum to 1."""
    rng = np.random.default_rng(7)
    x, wg, _, _ = rand_layer(rng, 64, 32, 16, 4)
    r = oracle.route(x, wg, 4)
    np.testing.assert_allclose(r.scores.astype(np.float64).sum(1), 1, atol=1e-6)
    sg = r.g.sum(1)
    assert (sg >= 4 / 16 - 1e-7).all() and (sg <= 1 + 1e-7).all()
    r_all = oracle.route(x, wg, 16)
    np.testing.assert_allclose(r_all.g.sum(1), 1, atol=1e-6)
    r_n = oracle.route(x, wg, 4, score="sigmoid", norm_topk=True)
    np.testing.assert_allclose(r_n.g.sum(1), 1, atol=1e-12)
    r_s = oracle.route(x, wg, 4, routed_scale=2.5)
    np.testing.assert_allclose(r_s.g, 2.5 * r.g, rtol=1e-15)


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def test_dense_reduction():
    """mN = mK = 1 and K_s = 0: the gate weight is exactly 1 and the layer is
    the residual plus one dense SwiGLU FFN (checked with torch)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(8)
    x, wg, routed, _ = rand_layer(rng, 10, 12, 1, 20)
    y, r = oracle.moe_forward(x, wg, routed, None, 1)
    assert (r.g == 1.0).all() and (r.idx == 0).all()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    w1, w3, w2 = (T(w[0]) for w in routed)
    want = T(x) + F.linear(F.silu(F.linear(T(x), w1)) * F.linear(T(x), w3), w2)
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-12)


def test_fine_grained_segmentation_identity():
    """One expert of inner I cut into m experts of inner I/m (row blocks of
    W1/W3, column blocks of W2).  With a zero gate every score is 1/m, and
    with all m kept the layer gives u + FFN_full(u) / m."""
    rng = np.random.default_rng(9)
    d, I, m = 16, 24, 4
    x = rng.standard_normal((7, d))
    w1 = rng.standard_normal((I, d)); w3 = rng.standard_normal((I, d))
    w2 = rng.standard_normal((d, I))
    blk = I // m
    routed = (np.stack([w1[i * blk:(i + 1) * blk] for i in range(m)]),
              np.stack([w3[i * blk:(i + 1) * blk] for i in range(m)]),
              np.stack([w2[:, i * blk:(i + 1) * blk] for i in range(m)]))
    y, r = oracle.moe_forward(x, np.zeros((m, d)), routed, None, m)
    np.testing.assert_allclose(r.g, 1.0 / m, rtol=1e-7)
    full = np.zeros((7, d))
    for t in range(7):       # dense FFN, written out row by row
        a = w1 @ x[t]; b = w3 @ x[t]
        full[t] = w2 @ (a / (1 + np.exp(-a)) * b)
    np.testing.assert_allclose(y, x + full * r.g[:, :1], rtol=1e-11, atol=1e-11)


def test_shared_concat_identity():
    """K_s shared experts of inner I act like one shared expert of inner
    K_s * I (W1/W3 rows and W2 columns concatenated)."""
    rng = np.random.default_rng(10)
    x, wg, routed, shared = rand_layer(rng, 9, 16, 4, 8, Ks=3, Is=6)
    y1, _ = oracle.moe_forward(x, wg, routed, shared, 2, n_shared=3)
    cat = (shared[0].reshape(1, 18, 16), shared[1].reshape(1, 18, 16),
           np.concatenate(list(shared[2]), axis=1)[None])
    y2, _ = oracle.moe_forward(x, wg, routed, cat, 2, n_shared=1)
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12)


def test_zero_down_projection_gives_residual_exactly():
    """All W2 = 0: every expert outputs 0 and y equals x bit for bit."""
    rng = np.random.default_rng(11)
    x, wg, routed, shared = rand_layer(rng, 9, 16, 6, 8, Ks=2)
    routed = (routed[0], routed[1], np.zeros_like(routed[2]))
    shared = (shared[0], shared[1], np.zeros_like(shared[2]))
    y, _ = oracle.moe_forward(x, wg, routed, shared, 3, n_shared=2)
    assert np.array_equal(y, x)


def test_shared_experts_always_active_with_unit_weight():
    """Routed experts off (W2 = 0): y = u + sum of shared FFNs, whatever the
    gate says -- shared experts take no gate weight."""
    rng = np.random.default_rng(12)
    x, wg, routed, shared = rand_layer(rng, 9, 16, 6, 8, Ks=2, Is=5)
    routed = (routed[0], routed[1], np.zeros_like(routed[2]))
    y, _ = oracle.moe_forward(x, wg * 50, routed, shared, 3, n_shared=2)
    want = x.copy()
    for s in range(2):
        for t in range(9):
            a = shared[0][s] @ x[t]; b = shared[1][s] @ x[t]
            want[t] += shared[2][s] @ (a / (1 + np.exp(-a)) * b)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("variant", [
    dict(),
    dict(score="sigmoid", select_bias=True, n_groups=4, topk_groups=2,
         norm_topk=True),
    dict(logit_bias=True),
    dict(routed_scale=2.5),
])
def test_bruteforce_equals_vectorised(variant):
    """Token-by-token loops with full sorts agree with the grouped oracle on
    the tiny workload and its routing variants."""
    inp = workloads.make_inputs("tiny-fp32")
    cfg = inp.cfg
    x, wg = inp.x()[:24], inp.w_gate()
    kw = dict(variant)
    rng = np.random.default_rng(13)
    if kw.pop("select_bias", False):
        kw["select_bias"] = (rng.random(cfg.n_routed) * 0.2 - 0.1).astype(np.float32)
    if kw.pop("logit_bias", False):
        kw["logit_bias"] = (-1.2 * np.log(rng.permutation(cfg.n_routed) + 1.0)).astype(np.float32)
    y, r = oracle.moe_forward(x, wg, inp.routed, inp.shared, cfg.top_k,
                              n_shared=cfg.n_shared, **kw)
    yb = oracle.moe_forward_bruteforce(x, wg, inp.routed, inp.shared,
                                       cfg.top_k, n_shared=cfg.n_shared, **kw)
    assert r.margin.min() > 1e-6     # no near-tie on this seed
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-9)


def test_mac_count_closed_form():
    """The multiply-adds the oracle performs equal T (d mN + 3 d (mK I +
    K_s I_s)): exactly mK routed and all K_s shared experts per token."""
    rng = np.random.default_rng(14)
    T, d, E, I, K, Ks, Is = 33, 16, 8, 12, 3, 2, 10
    x, wg, routed, shared = rand_layer(rng, T, d, E, I, Ks=Ks, Is=Is)
    stats = {}
    oracle.moe_forward(x, wg, routed, shared, K, n_shared=Ks, stats=stats)
    assert stats["macs"] == T * oracle.activated_macs_per_token(d, E, K, I, Ks, Is)
    # The expert FLOPs the benchmark prices are 2 per multiply-add the oracle
    # actually performed in the experts: its counter minus the gate's T d mN.
    for (T2, K2, Ks2) in ((T, K, Ks), (17, 1, 0), (9, E, 1)):
        x2, wg2, r2, s2 = rand_layer(rng, T2, d, E, I, Ks=max(Ks2, 1), Is=Is)
        st = {}
        oracle.moe_forward(x2, wg2, r2, s2, K2, n_shared=Ks2, stats=st)
        expert_macs = st["macs"] - T2 * d * E
        assert expert_macs % T2 == 0
        assert oracle.expert_flops_per_token(d, K2, I, Ks2, Is) == 2 * expert_macs // T2


def test_page_parameter_counts():
    """The pages' parameter totals fix the expert shapes the workloads use.

    16B: the 27 MoE layers hold (64 - 6) inactive routed experts of three
    2048 x 1408 matrices each: 13.55B, matching 16.4B total - 2.8B activated
    within the pages' rounding.  V3: (671 - 37)B inactive over 248 inactive
    experts of three 7168 x 2048 matrices gives about 58 MoE layers, no more
    than the 61 layers the report states.  16.4B 16-bit parameters fit the
    40 GB GPU named for deployment."""
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        pages = json.load(f)
    m16 = pages["deepseekmoe_16b"]
    c16 = workloads.CONFIGS["deepseekmoe-16b"]
    assert (c16.d, c16.n_routed, c16.n_shared, c16.top_k) == (
        m16["hidden"], m16["routed_experts"], m16["shared_experts"],
        m16["routed_per_token"])
    moe_layers = m16["transformer_layers"] - 1
    inactive = moe_layers * (c16.n_routed - c16.top_k) * 3 * c16.d * c16.inner
    want = (m16["total_params_billion"] - m16["activated_params_billion"]) * 1e9
    assert abs(inactive - want) / want < 0.01
    assert m16["total_params_billion"] * 1e9 * 2 < m16["deploy_gpu_memory_gb"] * 1e9
    v3 = pages["deepseek_v3"]
    c4 = workloads.CONFIGS["deepseek-v3"]
    assert (c4.n_routed, c4.top_k) == (v3["routed_experts"], v3["routed_per_token"])
    per_layer = (c4.n_routed - c4.top_k) * 3 * c4.d * c4.inner
    layers = (v3["total_params_billion"] - v3["activated_params_billion"]) * 1e9 / per_layer
    assert 55 <= layers <= v3["transformer_layers"]
    m2 = pages["deepseekmoe_2b"]
    c2 = workloads.CONFIGS["deepseekmoe-2b"]
    assert (c2.n_routed, c2.n_shared, c2.top_k) == (
        m2["routed_experts"], m2["shared_experts"], m2["routed_per_token"])


def test_token_permutation_equivariance():
    rng = np.random.default_rng(15)
    x, wg, routed, shared = rand_layer(rng, 20, 16, 8, 6, Ks=1)
    y, r = oracle.moe_forward(x, wg, routed, shared, 3, n_shared=1)
    p = rng.permutation(20)
    yp, rp = oracle.moe_forward(x[p], wg, routed, shared, 3, n_shared=1)
    np.testing.assert_allclose(yp, y[p], rtol=1e-13, atol=1e-13)
    assert np.array_equal(rp.idx, r.idx[p])


def test_expert_relabel_invariance():
    """Relabelling the routed experts (gate rows, weights, biases together)
    relabels the chosen indices and leaves y unchanged."""
    rng = np.random.default_rng(16)
    x, wg, routed, shared = rand_layer(rng, 20, 16, 8, 6, Ks=1)
    b = (rng.random(8) * 0.2).astype(np.float32)
    kw = dict(n_shared=1, score="sigmoid", select_bias=b, n_groups=2,
              topk_groups=1, norm_topk=True)
    # relabel inside each group so the group structure is preserved
    perm = np.concatenate([rng.permutation(4), 4 + rng.permutation(4)])
    y, r = oracle.moe_forward(x, wg, routed, shared, 3, **kw)
    kw["select_bias"] = b[perm]
    y2, r2 = oracle.moe_forward(x, wg[perm], tuple(w[perm] for w in routed),
                                shared, 3, **kw)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-13)
    assert np.array_equal(np.sort(perm[r2.idx], 1), np.sort(r.idx, 1))


# ---------------------------------------------------------------------------
# Dispatch bookkeeping
# ---------------------------------------------------------------------------

def test_dispatch_against_loops():
    """Counts, offsets and the (expert, token)-ordered rows, built with plain
    loops; every (token, slot) pair is placed exactly once (dropless)."""
    rng = np.random.default_rng(17)
    T, E, K = 50, 9, 3
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    dsp = oracle.dispatch(idx, E)
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            counts[idx[t, k]] += 1
    assert list(dsp.counts) == counts and dsp.counts.sum() == T * K
    rows = [(e, t) for e in range(E) for t in range(T) if e in idx[t]]
    assert list(dsp.row_src) == [t for _, t in rows]
    off = 0
    for e in range(E):
        assert dsp.offsets[e] == off
        off += counts[e]
    assert dsp.offsets[E] == T * K
    for t in range(T):
        for k in range(K):
            row = dsp.slot_row[t, k]
            assert dsp.row_src[row] == t
            assert dsp.offsets[idx[t, k]] <= row < dsp.offsets[idx[t, k] + 1]
    assert sorted(dsp.slot_row.ravel()) == list(range(T * K))
