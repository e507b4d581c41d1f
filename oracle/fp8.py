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


# Finite non-negative E4M3 values in code order (codes 0x00..0x7E increase
# with the value).
_MAGS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code to each value (|v| <= 448 expected), ties to the even
    code.  The sign of zero is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 0, 0x7E)   # first mag >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_MAGS[hi] - a)
    d_lo = np.abs(a - _MAGS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
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


def fp8_ffn(a_deq, w1q, w3q, w2q, quantize_h: bool = True) -> np.ndarray:
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
                    routed_scale: float = 1.0, forced_idx=None, quantize_h: bool = True):
    """The FP8 layer.  ``routed_q`` / ``shared_q`` are the results of
    ``quantize_experts`` (((codes, scales) for w1, w3, w2), stacked per expert).
    Routing is the bf16 layer's (on the input rows); the experts see the
    quantised token rows.  Returns (y [T, d] fp64, Routing)."""
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
        y += fp8_ffn(xd, *expert(shared_q, s_i), quantize_h=quantize_h)
    contrib = np.zeros((T, top_k, d))
    for e in np.unique(r.idx):
        tt, kk = np.nonzero(r.idx == e)
        contrib[tt, kk] = fp8_ffn(xd[tt], *expert(routed_q, int(e)), quantize_h=quantize_h)
    for k in range(top_k):
        y += r.g[:, k, None] * contrib[:, k]
    return y, r
