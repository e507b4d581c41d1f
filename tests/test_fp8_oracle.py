"""Pins of the FP8 (E4M3) oracle against the format's own definition and
constants and against properties any correct quantiser has.

The E4M3 constants below are those of the OCP 8-bit floating point format
(E4M3: exponent bias 7, largest finite 448 = 1.75 x 2^8, smallest normal 2^-6,
smallest subnormal 2^-9, S.1111.111 NaN, no infinities).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import fp8


def test_published_constants():
    v = fp8.e4m3_decode([0x7E, 0x08, 0x07, 0x01, 0x38, 0x00, 0x80, 0xFE, 0x40, 0x3C])
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 7 * 2.0 ** -9
    assert v[3] == 2.0 ** -9 and v[4] == 1.0 and v[5] == 0.0
    assert v[6] == 0.0 and math.copysign(1, v[6]) == -1.0
    assert v[7] == -448.0 and v[8] == 2.0 and v[9] == 1.5
    assert np.isnan(fp8.e4m3_decode([0x7F, 0xFF])).all()
    finite = fp8.e4m3_decode(np.arange(256))
    assert np.sum(~np.isnan(finite)) == 254


def test_code_order_and_round_trip():
    mags = fp8.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(mags) > 0)                 # codes increase with value
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_is_the_nearest_value_brute_force():
    """The encoder against a plain search of the 127 finite magnitudes: the
    nearest one, the even code on a tie."""
    mags = fp8.e4m3_decode(np.arange(0x7F))
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 4000),
                        rng.uniform(-0.05, 0.05, 4000),
                        (mags[1:] + mags[:-1]) / 2,                 # every midpoint
                        -(mags[1:] + mags[:-1]) / 2])
    got = fp8.e4m3_encode(v)
    for x, c in zip(v, got):
        dist = np.abs(mags - abs(x))
        best = np.flatnonzero(dist == dist.min())
        want = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        assert (int(c) & 0x7F) == want and (int(c) >> 7) == int(np.signbit(x)), x


def test_round_to_nearest_ties_to_even():
    enc = lambda x: int(fp8.e4m3_encode([x])[0])
    assert enc(1.0625) == 0x38            # midpoint of 1 (0x38) and 1.125 (0x39): even
    assert enc(1.1875) == 0x3A            # midpoint of 1.125 and 1.25 (0x3A): even
    assert enc(np.nextafter(1.0625, 2)) == 0x39
    assert enc(np.nextafter(1.0625, 0)) == 0x38
    assert enc(2.0 ** -10) == 0x00        # half the smallest subnormal: even (zero)
    assert enc(3 * 2.0 ** -10) == 0x02    # between 2^-9 (0x01) and 2^-8 (0x02): even
    assert enc(-1.0) == 0xB8 and enc(-0.0) == 0x80
    assert enc(440.0) == 0x7E and enc(416.0) == 0x7D   # 416 = 1.625 x 2^8


def test_scale_is_the_smallest_power_of_two():
    for amax in [448.0, 449.0, 1.0, 224.0, 224.5, 0.001, 3.7e5, 2.0 ** -100]:
        E = fp8.pow2_exponent(amax)
        assert amax <= 448.0 * 2.0 ** E
        assert amax > 448.0 * 2.0 ** (E - 1)
    assert fp8.pow2_exponent(0.0) == 0
    assert fp8.pow2_exponent(1e-300) == -127          # clamped to the byte range


def test_quantize_1x128_error_bounds():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((7, 512)) * np.exp(rng.uniform(-8, 8, (7, 1)))
    a[3, 128:256] = 0.0
    codes, sc = fp8.quantize_1x128(a)
    assert codes.dtype == np.uint8 and sc.shape == (7, 4)
    back = fp8.dequantize_1x128(codes, sc)
    E = sc.astype(np.int64) - 127
    for r in range(7):
        for g in range(4):
            blk = a[r, 128 * g:128 * (g + 1)]
            scaled = np.abs(blk) * 2.0 ** -E[r, g]
            if blk.any():
                assert 224.0 < scaled.max() <= 448.0          # range well used
            err = np.abs(back[r, 128 * g:128 * (g + 1)] - blk)
            normal = scaled >= 2.0 ** -6
            # half an ulp: 2^-4 relative for normals, 2^-10 absolute (scaled) below
            assert np.all(err[normal] <= np.abs(blk[normal]) * 2.0 ** -4)
            assert np.all(err[~normal] * 2.0 ** -E[r, g] <= 2.0 ** -10)
    assert np.all(back[3, 128:256] == 0.0) and sc[3, 1] == 127


def test_quantize_blocks_one_scale_per_block():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((256, 384))
    w[:128, 128:256] *= 1000.0
    codes, sc = fp8.quantize_blocks(w)
    assert sc.shape == (2, 3)
    assert sc[0, 1] - sc[0, 0] >= 9                     # 1000x larger block, >= 2^9
    back = fp8.dequantize_blocks(codes, sc)
    for i in range(2):
        for j in range(3):
            E = int(sc[i, j]) - 127
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            err = np.abs(back[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)] - blk)
            assert 224.0 < np.abs(blk).max() * 2.0 ** -E <= 448.0
            # half an ulp: 2^-4 relative, or 2^-10 of the scale below the normals
            assert np.all(err <= np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** (E - 10)))


def test_exactly_representable_inputs_survive_quantisation():
    """Values already of the form code x 2^k with the group maximum using the
    scale fully come back bitwise."""
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 0x7F, (4, 256)).astype(np.uint8)
    codes[:, 0] = 0x7E                                    # each group reaches 448 ...
    codes[:, 128] = 0x7E
    a = fp8.e4m3_decode(codes) * 2.0 ** -5                # ... times 2^-5
    q, sc = fp8.quantize_1x128(a)
    assert np.all(sc == 127 - 5) and np.array_equal(q, codes)


def test_fp8_layer_without_h_quantisation_is_the_layer_on_quantised_operands():
    """With the H quantiser switched off the FP8 layer must equal the bf16
    layer's oracle run on the dequantised token rows and weights (the layer
    wiring: which operand is quantised how, shared and routed paths)."""
    rng = np.random.default_rng(3)
    T, d, E, I, K = 40, 256, 8, 128, 2
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / 16
    w1 = rng.standard_normal((E, I, d)) / 16
    w3 = rng.standard_normal((E, I, d)) / 16
    w2 = rng.standard_normal((E, d, I)) / 11
    s1, s3, s2 = (rng.standard_normal((1,) + w.shape[1:]) / 16 for w in (w1, w3, w2))
    rq = fp8.quantize_experts(w1, w3, w2)
    sq = fp8.quantize_experts(s1, s3, s2)
    # A zero gate gives every expert the same score for x and for its
    # quantised rows, so both runs weigh the forced choices identically.
    wg = np.zeros_like(wg)
    forced = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    y, r = fp8.moe_forward_fp8(x, wg, rq, sq, K, n_shared=1, quantize_h=False,
                               forced_idx=forced)
    deq = lambda q: np.stack([fp8.dequantize_blocks(q[0][e], q[1][e]) for e in range(q[0].shape[0])])
    xd = fp8.dequantize_1x128(*fp8.quantize_1x128(x))
    want, _ = oracle.moe_forward(xd, wg, tuple(deq(q) for q in rq), tuple(deq(q) for q in sq),
                                 K, n_shared=1, forced_idx=forced)
    want += x - xd                                        # the residual is the unquantised x
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r.idx, forced)


def test_fp8_layer_error_against_bf16_layer_is_quantisation_sized():
    rng = np.random.default_rng(4)
    T, d, E, I, K = 64, 256, 8, 128, 2
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / 16
    w1 = rng.standard_normal((E, I, d)) / 16
    w3 = rng.standard_normal((E, I, d)) / 16
    w2 = rng.standard_normal((E, d, I)) / 11
    y8, _ = fp8.moe_forward_fp8(x, wg, fp8.quantize_experts(w1, w3, w2), None, K)
    y, _ = oracle.moe_forward(x, wg, (w1, w3, w2), None, K)
    rel = np.sqrt(np.mean((y8 - y) ** 2)) / np.sqrt(np.mean((y - x) ** 2))
    assert 0.01 < rel < 0.15       # E4M3 keeps 3 mantissa bits: a few percent


def _requant(h):
    return fp8.dequantize_1x128(*fp8.quantize_1x128(h))


def test_requantisation_spread_bounds_every_move():
    """``requantisation_spread`` against brute force: random moves of every
    value by at most margin x its group's maximum never change the quantised
    value by more than the spread; moving a whole group by +/- the margin
    reaches it where the scale cannot change; zero margin gives zero."""
    rng = np.random.default_rng(11)
    h = rng.standard_normal((6, 384)) * np.exp(rng.uniform(-6, 6, (6, 1)))
    h[0, :128] *= 56.0 / np.abs(h[0, :128]).max()         # max exactly 448 x 2^-3
    h[1, 128:256] = 0.0                                   # a group of zeros ...
    h[1, 130] = 1e-3                                      # ... but one tiny value
    h[2, 256:] *= 1e-4                                    # tiny values: subnormal codes
    v = _requant(h)
    assert np.array_equal(fp8.requantisation_spread(h, 0.0), np.zeros_like(h))
    margin = 1e-3
    spread = fp8.requantisation_spread(h, margin)
    R, C = h.shape
    gmax = np.abs(h.reshape(R, C // 128, 128)).max(2)
    delta = np.repeat(margin * gmax, 128, axis=1)
    worst = np.zeros_like(h)
    moves = [np.full_like(h, 1.0), np.full_like(h, -1.0)]
    moves += [rng.uniform(-1, 1, h.shape) for _ in range(300)]
    moves += [np.sign(rng.uniform(-1, 1, h.shape)) for _ in range(100)]
    for m in moves:
        dev = np.abs(_requant(h + m * delta) - v)
        assert np.all(dev <= spread * (1 + 1e-12)), np.argwhere(dev > spread)[0]
        worst = np.maximum(worst, dev)
    # the group on the scale boundary: moving up changes its scale
    assert fp8.quantize_1x128(h + delta)[1][0, 0] == fp8.quantize_1x128(h)[1][0, 0] + 1
    # where the scale is fixed the two uniform moves attain the spread
    E = lambda a: np.repeat(fp8.quantize_1x128(a)[1], 128, axis=1)
    fixed = (E(h + delta) == E(h)) & (E(h - delta) == E(h))
    fixed &= np.repeat(np.abs(gmax) * (1 + margin) < 448.0 * np.exp2(
        fp8.quantize_1x128(h)[1].astype(np.int64) - 127), 128, axis=1)
    fixed &= np.repeat(np.abs(gmax) * (1 - margin) > 224.0 * np.exp2(
        fp8.quantize_1x128(h)[1].astype(np.int64) - 127), 128, axis=1)
    assert fixed.sum() > 0.5 * h.size
    np.testing.assert_array_equal(worst[fixed], spread[fixed])
    # tiny values near zero: a move can flip the sign of a subnormal code
    assert spread[1, 131] > 0 and spread[1, 131] <= 2 * margin * 1e-3
