"""FP8 (E4M3) variant of the layer: quantisers and the forward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): shares no code with the
HIP library.

What the pages fix (DeepSeek-V3 Technical Report summary, "3.3 FP8 Training"
and "B.2 Discussion About Block-Wise Quantization"): most GEMMs run in FP8 with
fine-grained scaling and high-precision accumulation; activations are scaled
per 1x128 group along the GEMM's reduction dimension (unlike 128x128 blocks);
activations quantised before the MoE dispatch use power-of-two scaling
factors.  Readings where the pages are silent: the element format is OCP E4M3
(4 exponent bits, bias 7, 3 mantissa bits, subnormals, no infinities, one NaN
pattern per sign); weights are scaled per 128x128 block; every scale is a
power of two (an 8-bit exponent, value 2^(byte - 127)), the smallest one that
keeps the group's largest magnitude within E4M3's largest finite value 448;
values are rounded to the nearest E4M3 value, ties to the even code.

The layer: the router is unchanged (fp32 gate on the input rows); each
expert's two GEMMs take FP8 operands -- the token rows quantised per 1x128 of
the hidden dimension, the SwiGLU activations H per 1x128 of the inner
dimension, the weights as given (codes + block exponents) -- and accumulate
exactly (fp64 here); the residual and the combine are as in the bf16 layer.
"""
from __future__ import annotations

import math

import numpy as np

from .moe_oracle import route, silu

E4M3_MAX = 448.0
GROUP = 128


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code: (-1)^S * 2^(E-7) * (1 + M/8) for E >= 1,
    (-1)^S * 2^-6 * M/8 for E = 0; S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = s * v
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code to each value (|v| <= 448 expected), ties to the even
    code.  The sign of zero is kept.

    Normal range (|v| >= 2^-6): |v| = q 2^e with q in [1, 2); the 3-bit
    mantissa is q rounded to a multiple of 1/8 (numpy's rint: half to even),
    a round-up to 2 carrying into the exponent.  Below 2^-6 the values are the
    multiples of 2^-9, rounded the same way (8 x 2^-9 is the smallest normal,
    whose code is 8).  Codes increase with the value, so the even code is the
    even mantissa."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # a = q 2^e, q in [1, 2): the exponent and significand fields of the fp64
    # value (exact; only used where a >= 2^-6, i.e. a is a normal fp64)
    bits = a.view(np.int64)
    e = ((bits >> 52) & 0x7FF) - 1023
    q = ((bits & 0xFFFFFFFFFFFFF) | (1023 << 52)).view(np.float64)
    m = np.rint((q - 1.0) * 8.0)
    carry = m == 8.0
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0.0, m)
    normal = (e + 7) * 8 + m
    sub = np.rint(a * 512.0)
    code = np.where(a >= 2.0 ** -6, normal, sub)
    code = np.clip(code, 0, 0x7E).astype(np.int64)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def pow2_exponent(amax: float) -> int:
    """The smallest integer E with amax <= 448 * 2^E, in [-127, 127]; 0 for a
    group of zeros."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    E = math.frexp(amax)[1] - 9              # a first guess, then the definition
    while amax > E4M3_MAX * 2.0 ** E:
        E += 1
    while amax <= E4M3_MAX * 2.0 ** (E - 1):
        E -= 1
    return max(-127, min(127, E))


def quantize_1x128(a):
    """Rows of ``a`` [R][C] (C a multiple of 128) in E4M3 with one power-of-two
    scale per 128 consecutive columns of a row.  Returns (codes uint8 [R][C],
    scale bytes uint8 [R][C/128], byte = E + 127)."""
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    g = a.reshape(R, C // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    E = np.vectorize(pow2_exponent, otypes=[np.int64])(amax) if amax.size else \
        np.zeros(amax.shape, np.int64)
    codes = e4m3_encode(g * np.exp2(-E)[:, :, None]).reshape(R, C)
    return codes, (E + 127).astype(np.uint8)


def quantize_blocks(w):
    """A matrix ``w`` [R][C] (multiples of 128) in E4M3 with one power-of-two
    scale per 128x128 block.  Returns (codes [R][C], scale bytes [R/128][C/128])."""
    w = np.asarray(w, dtype=np.float64)
    R, C = w.shape
    b = w.reshape(R // GROUP, GROUP, C // GROUP, GROUP)
    amax = np.abs(b).max(axis=(1, 3))
    E = np.vectorize(pow2_exponent, otypes=[np.int64])(amax)
    codes = e4m3_encode(b * np.exp2(-E)[:, None, :, None]).reshape(R, C)
    return codes, (E + 127).astype(np.uint8)


def dequantize_1x128(codes, scales) -> np.ndarray:
    v = e4m3_decode(codes)
    R, C = v.shape
    return (v.reshape(R, C // GROUP, GROUP) *
            np.exp2(np.asarray(scales, np.float64) - 127.0)[:, :, None]).reshape(R, C)


def dequantize_blocks(codes, scales) -> np.ndarray:
    v = e4m3_decode(codes)
    R, C = v.shape
    s = np.exp2(np.asarray(scales, np.float64) - 127.0)
    return (v.reshape(R // GROUP, GROUP, C // GROUP, GROUP) *
            s[:, None, :, None]).reshape(R, C)


def quantize_experts(w1, w3, w2):
    """Stacked expert weights (w1, w3 [E][I][d], w2 [E][d][I]) as E4M3 codes
    and 128x128 block scale bytes, per expert."""
    out = []
    for w in (w1, w3, w2):
        q = [quantize_blocks(w[e]) for e in range(w.shape[0])]
        out.append((np.stack([c for c, _ in q]), np.stack([s for _, s in q])))
    return tuple(out)


def requantisation_spread(h, margin: float) -> np.ndarray:
    """How far the 1x128 quantisation of ``h`` [R][C] can move if every value
    moves by at most ``margin`` times its group's largest magnitude: for each
    element, the largest |Q(h') - Q(h)| over such h', where Q quantises and
    dequantises as ``quantize_1x128`` does (the scale chosen from the moved
    group's own maximum).

    Q is monotone in each value for a fixed scale, so the extremes are taken
    at h -/+ delta, under every scale exponent the moved maximum (within
    delta of the original) can pick."""
    h = np.asarray(h, np.float64)
    R, C = h.shape
    g = h.reshape(R, C // GROUP, GROUP)
    gmax = np.abs(g).max(axis=2)
    delta = margin * gmax
    pe = np.vectorize(pow2_exponent, otypes=[np.int64])
    if gmax.size == 0:
        return np.zeros_like(h)
    E_lo = pe(np.maximum(gmax - delta, 0.0))
    E_hi = pe(gmax + delta)
    E0 = pe(gmax)
    v = dequantize_1x128(*quantize_1x128(h)).reshape(R, C // GROUP, GROUP)
    spread = np.zeros_like(g)
    for dE in range(int((E_lo - E0).min()), int((E_hi - E0).max()) + 1):
        E = E0 + dE
        live = (E >= E_lo) & (E <= E_hi)
        sc = np.exp2(E.astype(np.float64))[:, :, None]
        for sgn in (-1.0, 1.0):
            moved = np.clip((g + sgn * delta[:, :, None]) / sc, -E4M3_MAX, E4M3_MAX)
            q = e4m3_decode(e4m3_encode(moved)) * sc
            spread = np.where(live[:, :, None], np.maximum(spread, np.abs(q - v)), spread)
    return spread.reshape(R, C)


def fp8_ffn(a_deq, w1q, w3q, w2q, quantize_h: bool = True, h_margin=None):
    """One expert on FP8 operands: token rows ``a_deq`` (already quantised
    per 1x128 and dequantised), weights (codes, block scales).  H is quantised
    per 1x128 of the inner dimension before the down-projection (skipped with
    ``quantize_h=False``).  Accumulation is exact (fp64).

    With ``h_margin`` also returns, per output element, the largest change
    that moving H by ``h_margin`` of its groups' maxima before quantising it
    (``requantisation_spread``) can make to it."""
    W1 = dequantize_blocks(*w1q)
    W3 = dequantize_blocks(*w3q)
    W2 = dequantize_blocks(*w2q)
    h = silu(a_deq @ W1.T) * (a_deq @ W3.T)
    allow = None
    if quantize_h:
        if h_margin is not None:
            allow = requantisation_spread(h, h_margin) @ np.abs(W2).T
        h = dequantize_1x128(*quantize_1x128(h))
    y = h @ W2.T
    if h_margin is None:
        return y
    return y, (allow if allow is not None else np.zeros_like(y))


def moe_forward_fp8(x, w_gate, routed_q, shared_q, top_k: int, *, n_shared: int = 0,
                    score: str = "softmax", logit_bias=None, select_bias=None,
                    n_groups: int = 1, topk_groups: int = 1, norm_topk: bool = False,
                    routed_scale: float = 1.0, forced_idx=None, quantize_h: bool = True,
                    h_margin=None):
    """The FP8 layer.  ``routed_q`` / ``shared_q`` are the results of
    ``quantize_experts`` (((codes, scales) for w1, w3, w2), stacked per expert).
    Routing is the bf16 layer's (on the input rows); the experts see the
    quantised token rows.  Returns (y [T, d] fp64, Routing), and with
    ``h_margin`` also, per output element, the largest change that moving
    each expert's H by ``h_margin`` of its 1x128 groups' maxima can make
    (weighted like the experts' contributions)."""
    x64 = np.asarray(x, np.float64)
    T, d = x64.shape
    r = route(x, w_gate, top_k, score=score, logit_bias=logit_bias,
              select_bias=select_bias, n_groups=n_groups, topk_groups=topk_groups,
              norm_topk=norm_topk, routed_scale=routed_scale, forced_idx=forced_idx)
    xd = dequantize_1x128(*quantize_1x128(x64))

    def expert(q, e):
        (c1, s1), (c3, s3), (c2, s2) = q
        return (c1[e], s1[e]), (c3[e], s3[e]), (c2[e], s2[e])

    track = h_margin is not None
    allow = np.zeros((T, d))
    y = x64.copy()
    for s_i in range(n_shared):
        out = fp8_ffn(xd, *expert(shared_q, s_i), quantize_h=quantize_h, h_margin=h_margin)
        if track:
            out, a = out
            allow += a
        y += out
    contrib = np.zeros((T, top_k, d))
    c_allow = np.zeros((T, top_k, d)) if track else None
    for e in np.unique(r.idx):
        tt, kk = np.nonzero(r.idx == e)
        out = fp8_ffn(xd[tt], *expert(routed_q, int(e)), quantize_h=quantize_h,
                      h_margin=h_margin)
        if track:
            out, a = out
            c_allow[tt, kk] = a
        contrib[tt, kk] = out
    for k in range(top_k):
        y += r.g[:, k, None] * contrib[:, k]
        if track:
            allow += np.abs(r.g[:, k, None]) * c_allow[:, k]
    return (y, r, allow) if track else (y, r)
