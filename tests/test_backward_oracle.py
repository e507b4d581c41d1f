"""Pins of the backward oracle (``oracle.moe_backward``) against things other
than itself: central finite differences of the exact forward, torch.autograd
(fp64, CPU) of a plain torch forward written here, and closed-form cases."""
import numpy as np
import pytest
import torch

import oracle


def _layer(rng, T, d, E, I, K, Ks, Is=None):
    Is = Is or I
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / np.sqrt(d)
    routed = (rng.standard_normal((E, I, d)) / np.sqrt(d),
              rng.standard_normal((E, I, d)) / np.sqrt(d),
              rng.standard_normal((E, d, I)) / np.sqrt(I))
    shared = None
    if Ks:
        shared = (rng.standard_normal((Ks, Is, d)) / np.sqrt(d),
                  rng.standard_normal((Ks, Is, d)) / np.sqrt(d),
                  rng.standard_normal((Ks, d, Is)) / np.sqrt(Is))
    return x, wg, routed, shared


VARIANTS = {
    "softmax": dict(score="softmax"),
    "softmax-scaled-bias": dict(score="softmax", routed_scale=2.5, logit_bias=True),
    "sigmoid-norm-groups": dict(score="sigmoid", norm_topk=True, n_groups=3, topk_groups=2,
                                select_bias=True),
}


def _kw(rng, E, v):
    kw = dict(v)
    if kw.pop("logit_bias", False):
        kw["logit_bias"] = rng.uniform(-1, 1, E)
    if kw.pop("select_bias", False):
        kw["select_bias"] = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return kw


@pytest.mark.parametrize("name", list(VARIANTS))
def test_backward_matches_central_differences(name):
    rng = np.random.default_rng(10)
    T, d, E, I, K, Ks = 4, 6, 6, 4, 2, 1
    x, wg, routed, shared = _layer(rng, T, d, E, I, K, Ks)
    kw = _kw(rng, E, VARIANTS[name])
    dy = rng.standard_normal((T, d))
    gr = oracle.moe_backward(x, wg, routed, shared, K, dy, n_shared=Ks, **kw)
    fkw = {k: v for k, v in kw.items() if k not in ("select_bias", "n_groups", "topk_groups")}

    def L(x_=x, wg_=wg, routed_=routed, shared_=shared, lb_=kw.get("logit_bias")):
        fk = dict(fkw)
        if lb_ is not None:
            fk["logit_bias"] = lb_
        y = oracle.moe_forward_exact(x_, wg_, routed_, shared_, K, n_shared=Ks,
                                     forced_idx=gr.idx, **fk)
        return float((dy * y).sum())

    eps = 1e-6

    def fd(arr, make):
        g = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a, b = arr.copy(), arr.copy()
            a[i] += eps
            b[i] -= eps
            g[i] = (make(a) - make(b)) / (2 * eps)
        return g

    np.testing.assert_allclose(gr.dx, fd(x, lambda a: L(x_=a)), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(gr.dw_gate, fd(wg, lambda a: L(wg_=a)), rtol=1e-6, atol=1e-8)
    if "logit_bias" in kw:
        np.testing.assert_allclose(gr.dlogit_bias, fd(kw["logit_bias"], lambda a: L(lb_=a)),
                                   rtol=1e-6, atol=1e-8)
    for j in range(3):
        def mk_r(a, j=j):
            w = list(routed)
            w[j] = a
            return L(routed_=tuple(w))

        def mk_s(a, j=j):
            w = list(shared)
            w[j] = a
            return L(shared_=tuple(w))
        np.testing.assert_allclose(gr.routed[j], fd(routed[j], mk_r), rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose(gr.shared[j], fd(shared[j], mk_s), rtol=1e-6, atol=1e-8)


def _torch_layer(x, wg, lb, routed, shared, idx, score, norm_topk, scale):
    """The layer written with torch ops (selection given), for autograd."""
    l = x @ wg.T
    if lb is not None:
        l = l + lb
    s = torch.softmax(l, dim=1) if score == "softmax" else torch.sigmoid(l)
    s_sel = torch.gather(s, 1, idx)
    g = s_sel / s_sel.sum(1, keepdim=True) if norm_topk else s_sel
    g = g * scale
    y = x.clone()
    if shared is not None:
        for si in range(shared[0].shape[0]):
            h = torch.nn.functional.silu(x @ shared[0][si].T) * (x @ shared[2 - 1][si].T)
            y = y + h @ shared[2][si].T
    for k in range(idx.shape[1]):
        e = idx[:, k]
        a1 = torch.einsum("td,tid->ti", x, routed[0][e])
        a3 = torch.einsum("td,tid->ti", x, routed[1][e])
        h = torch.nn.functional.silu(a1) * a3
        y = y + g[:, k:k + 1] * torch.einsum("ti,tdi->td", h, routed[2][e])
    return y


@pytest.mark.parametrize("name", list(VARIANTS))
def test_backward_matches_torch_autograd(name):
    rng = np.random.default_rng(11)
    T, d, E, I, K, Ks = 40, 16, 9, 8, 3, 2
    x, wg, routed, shared = _layer(rng, T, d, E, I, K, Ks, Is=12)
    kw = _kw(rng, E, VARIANTS[name])
    dy = rng.standard_normal((T, d))
    gr = oracle.moe_backward(x, wg, routed, shared, K, dy, n_shared=Ks, **kw)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, twg = t(x), t(wg)
    tlb = t(kw["logit_bias"]) if "logit_bias" in kw else None
    tr = tuple(t(w) for w in routed)
    ts = tuple(t(w) for w in shared)
    y = _torch_layer(tx, twg, tlb, tr, ts, torch.tensor(gr.idx, dtype=torch.int64),
                     kw.get("score", "softmax"), kw.get("norm_topk", False),
                     kw.get("routed_scale", 1.0))
    (y * torch.tensor(dy)).sum().backward()
    close = lambda a, b: np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-10, atol=1e-12)
    close(gr.dx, tx)
    close(gr.dw_gate, twg)
    if tlb is not None:
        close(gr.dlogit_bias, tlb)
    for j in range(3):
        close(gr.routed[j], tr[j])
        close(gr.shared[j], ts[j])


def test_zero_down_projection_passes_dy_through():
    """W2 = 0: every expert output is zero, so dx = dy exactly, the gate
    receives no gradient, and W1/W3 receive none."""
    rng = np.random.default_rng(12)
    x, wg, routed, shared = _layer(rng, 30, 8, 6, 4, 2, 1)
    routed = (routed[0], routed[1], np.zeros_like(routed[2]))
    shared = (shared[0], shared[1], np.zeros_like(shared[2]))
    dy = rng.standard_normal(x.shape)
    gr = oracle.moe_backward(x, wg, routed, shared, 2, dy, n_shared=1)
    assert np.array_equal(gr.dx, dy)
    assert not gr.dw_gate.any() and not gr.dlogit_bias.any()
    for w in gr.routed[:2] + gr.shared[:2]:
        assert not w.any()
    assert np.abs(gr.routed[2]).max() > 0


def test_single_expert_and_single_kept_normalised_have_no_router_gradient():
    rng = np.random.default_rng(13)
    x, wg, routed, shared = _layer(rng, 20, 8, 1, 4, 1, 0)
    dy = rng.standard_normal(x.shape)
    gr = oracle.moe_backward(x, wg, routed, None, 1, dy)       # softmax over one expert: s = 1
    assert not gr.dw_gate.any() and not gr.dlogits.any()
    x, wg, routed, shared = _layer(rng, 20, 8, 5, 4, 1, 0)
    gr = oracle.moe_backward(x, wg, routed, None, 1, dy, score="sigmoid", norm_topk=True)
    assert not gr.dw_gate.any()                                 # g = s / s = 1
    assert np.abs(gr.dg).max() > 0


def test_gate_weight_gradient_is_dy_dot_expert_output():
    """dg_{t,k} against the forward oracle's own expert output."""
    rng = np.random.default_rng(14)
    x, wg, routed, shared = _layer(rng, 25, 8, 6, 4, 2, 1)
    dy = rng.standard_normal(x.shape)
    gr = oracle.moe_backward(x, wg, routed, shared, 2, dy, n_shared=1)
    for t in range(25):
        for k in range(2):
            e = gr.idx[t, k]
            ye = oracle.swiglu_ffn(x[t:t + 1], routed[0][e], routed[1][e], routed[2][e])[0]
            assert abs(gr.dg[t, k] - dy[t] @ ye) <= 1e-12 * (1 + abs(dy[t] @ ye))


def test_magnitudes_bound_the_error_of_one_rounded_factor():
    """The reported sums of |terms| bound the change of each gradient when
    one factor of every term is rounded to bf16 (8 significant bits: a
    relative rounding error of at most 2^-8): the
    SwiGLU input gradients for dW1, dW3 and dx, g h for dW2 -- emulated here
    with torch's bf16 rounding -- and the bound is not loose by orders of
    magnitude."""
    rng = np.random.default_rng(15)
    x, wg, routed, shared = _layer(rng, 60, 16, 4, 8, 2, 1)
    dy = rng.standard_normal(x.shape)
    gr = oracle.moe_backward(x, wg, routed, shared, 2, dy, n_shared=1, magnitudes=True)
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    s = oracle.exact_scores(x, wg, None, "softmax")
    g = np.take_along_axis(s, gr.idx.astype(np.int64), 1)
    ratios = []
    for e in range(4):
        tt, kk = np.nonzero(gr.idx == e)
        u = x[tt]
        w1, w3, w2 = routed[0][e], routed[1][e], routed[2][e]
        a1, a3 = u @ w1.T, u @ w3.T
        sg = 1 / (1 + np.exp(-a1))
        h = a1 * sg * a3
        dh = g[tt, kk, None] * dy[tt] @ w2
        da1 = dh * a3 * sg * (1 + a1 * (1 - sg))
        da3 = dh * a1 * sg
        for got, ref, mag in ((bf(da1).T @ u, gr.routed[0][e], gr.routed_mag[0][e]),
                              (bf(da3).T @ u, gr.routed[1][e], gr.routed_mag[1][e]),
                              (dy[tt].T @ bf(g[tt, kk, None] * h), gr.routed[2][e],
                               gr.routed_mag[2][e])):
            err = np.abs(got - ref)
            assert np.all(err <= 2.0 ** -8 * mag + 1e-15)
            ratios.append((err / (2.0 ** -8 * mag)).max())
    assert max(ratios) > 0.3                     # and not loose
