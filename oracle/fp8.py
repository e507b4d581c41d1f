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


def _silu_argmin() -> float:
    """The point where silu(a) = a / (1 + e^-a) is smallest: the root of
    silu'(a) = sigmoid(a) (1 + a sigmoid(-a)), i.e. of 1 + a / (1 + e^a),
    by Newton's method from -1.3."""
    a = -1.3
    for _ in range(50):
        ea = math.exp(a)
        f = 1.0 + a / (1.0 + ea)
        df = (1.0 + ea - a * ea) / (1.0 + ea) ** 2
        step = f / df
        a -= step
        if abs(step) < 1e-17:
            break
    return a


SILU_ARGMIN = _silu_argmin()


def silu_range(lo, hi):
    """Smallest and largest value of silu over each interval [lo, hi]: silu
    falls on (-inf, SILU_ARGMIN] and rises after it."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    s_lo, s_hi = silu(lo), silu(hi)
    vmin = np.where((lo < SILU_ARGMIN) & (hi > SILU_ARGMIN), silu(SILU_ARGMIN),
                    np.minimum(s_lo, s_hi))
    return vmin, np.maximum(s_lo, s_hi)


def activation_interval(a_deq, W1, W3, acc_rel: float, eval_rel: float = 2.0 ** -20):
    """The SwiGLU activations h = silu(a1) * a3 of rows ``a_deq`` [R, d]
    (dequantised token rows) with dequantised weights W1, W3 [I, d], and for
    each one the interval [h_lo, h_hi] of values it can take when each
    pre-activation a = sum_j t_j (t_j = u_j W_j) is off by at most
    ``acc_rel`` * sum_j |t_j| (an accumulation that loses that much), widened
    by ``eval_rel`` of its largest magnitude for the evaluation of silu and
    the product in fp32.  Returns (h, h_lo, h_hi), each [R, I], fp64."""
    u = np.asarray(a_deq, np.float64)
    W1 = np.asarray(W1, np.float64)
    W3 = np.asarray(W3, np.float64)
    a1, a3 = u @ W1.T, u @ W3.T
    au = np.abs(u)
    d1 = acc_rel * (au @ np.abs(W1).T)
    d3 = acc_rel * (au @ np.abs(W3).T)
    s_lo, s_hi = silu_range(a1 - d1, a1 + d1)
    b_lo, b_hi = a3 - d3, a3 + d3
    p = np.stack([s_lo * b_lo, s_lo * b_hi, s_hi * b_lo, s_hi * b_hi])
    h_lo, h_hi = p.min(axis=0), p.max(axis=0)
    slack = eval_rel * np.maximum(np.abs(h_lo), np.abs(h_hi))
    return silu(a1) * a3, h_lo - slack, h_hi + slack


def admissible_1x128(h_lo, h_hi, codes, scales):
    """Is each given E4M3 code (with its 1x128 group's scale byte) the
    quantisation of some value inside its interval [h_lo, h_hi]?

    The group's scale must be one the quantiser can pick for some values
    inside the intervals: 2^E with E between the exponents of the largest
    smallest-magnitude and the largest largest-magnitude (E = 0 also allowed
    when every interval can be zero).  Given that scale, quantisation is
    monotone in the value, so the code must lie between the quantisations of
    the interval's two ends.  Returns (ok [R, C] bool, scale_ok [R, C/128]
    bool); ok is False wherever its group's scale is not admissible."""
    h_lo = np.asarray(h_lo, np.float64)
    h_hi = np.asarray(h_hi, np.float64)
    R, C = h_lo.shape
    G = C // GROUP
    mag_lo = np.where((h_lo <= 0) & (h_hi >= 0), 0.0, np.minimum(np.abs(h_lo), np.abs(h_hi)))
    mag_hi = np.maximum(np.abs(h_lo), np.abs(h_hi))
    m_lo = mag_lo.reshape(R, G, GROUP).max(axis=2)
    m_hi = mag_hi.reshape(R, G, GROUP).max(axis=2)
    pe = np.vectorize(pow2_exponent, otypes=[np.int64])
    E_lo = np.where(m_lo > 0, pe(m_lo), -127)
    E_hi = pe(m_hi)
    E = np.asarray(scales, np.int64) - 127
    scale_ok = ((E >= E_lo) & (E <= E_hi)) | ((m_lo == 0) & (E == 0))
    sc = np.repeat(np.exp2(E.astype(np.float64)), GROUP, axis=1)
    q = lambda v: e4m3_decode(e4m3_encode(np.clip(v / sc, -E4M3_MAX, E4M3_MAX))) * sc
    val = e4m3_decode(codes) * sc
    ok = (val >= q(h_lo)) & (val <= q(h_hi)) & np.repeat(scale_ok, GROUP, axis=1)
    return ok, scale_ok


def fp8_ffn(a_deq, w1q, w3q, w2q, quantize_h: bool = True):
    """One expert on FP8 operands: token rows ``a_deq`` (already quantised
    per 1x128 and dequantised), weights (codes, block scales).  H is quantised
    per 1x128 of the inner dimension before the down-projection (skipped with
    ``quantize_h=False``).  Accumulation is exact (fp64)."""
    W1 = dequantize_blocks(*w1q)
    W3 = dequantize_blocks(*w3q)
    W2 = dequantize_blocks(*w2q)
    h = silu(a_deq @ W1.T) * (a_deq @ W3.T)
    if quantize_h:
        h = dequantize_1x128(*quantize_1x128(h))
    return h @ W2.T


def moe_forward_fp8(x, w_gate, routed_q, shared_q, top_k: int, *, n_shared: int = 0,
                    score: str = "softmax", logit_bias=None, select_bias=None,
                    n_groups: int = 1, topk_groups: int = 1, norm_topk: bool = False,
                    routed_scale: float = 1.0, forced_idx=None, quantize_h: bool = True,
                    forced_h=None):
    """The FP8 layer.  ``routed_q`` / ``shared_q`` are the results of
    ``quantize_experts`` (((codes, scales) for w1, w3, w2), stacked per expert).
    Routing is the bf16 layer's (on the input rows); the experts see the
    quantised token rows.  Returns (y [T, d] fp64, Routing).

    ``forced_h`` = (shared [K_s][T][I_s], routed [T][K][I]) replaces the
    quantised SwiGLU activations (dequantised values) that enter the
    down-projections -- where the gate/up products admit several correct
    E4M3 codes, the layer is evaluated on a given admissible choice (see
    ``admissible_1x128``), as ``forced_idx`` does for the expert choice."""
    x64 = np.asarray(x, np.float64)
    T, d = x64.shape
    r = route(x, w_gate, top_k, score=score, logit_bias=logit_bias,
              select_bias=select_bias, n_groups=n_groups, topk_groups=topk_groups,
              norm_topk=norm_topk, routed_scale=routed_scale, forced_idx=forced_idx)
    xd = dequantize_1x128(*quantize_1x128(x64))

    def expert(q, e):
        (c1, s1), (c3, s3), (c2, s2) = q
        return (c1[e], s1[e]), (c3[e], s3[e]), (c2[e], s2[e])

    y = x64.copy()
    for s_i in range(n_shared):
        if forced_h is not None:
            W2 = dequantize_blocks(*expert(shared_q, s_i)[2])
            y += np.asarray(forced_h[0][s_i], np.float64) @ W2.T
        else:
            y += fp8_ffn(xd, *expert(shared_q, s_i), quantize_h=quantize_h)
    contrib = np.zeros((T, top_k, d))
    for e in np.unique(r.idx):
        tt, kk = np.nonzero(r.idx == e)
        if forced_h is not None:
            W2 = dequantize_blocks(*expert(routed_q, int(e))[2])
            contrib[tt, kk] = np.asarray(forced_h[1][tt, kk], np.float64) @ W2.T
        else:
            contrib[tt, kk] = fp8_ffn(xd[tt], *expert(routed_q, int(e)), quantize_h=quantize_h)
    for k in range(top_k):
        y += r.g[:, k, None] * contrib[:, k]
    return y, r
