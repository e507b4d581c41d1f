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


def test_silu_minimum_and_range_brute_force():
    """SILU_ARGMIN is where silu is smallest (a dense grid agrees, and the
    derivative vanishes there); silu_range over random intervals equals the
    extremes of silu on a dense sampling of each interval."""
    a = fp8.SILU_ARGMIN
    grid = np.linspace(-3.0, 1.0, 400001)
    sg = oracle.silu(grid)
    assert abs(grid[np.argmin(sg)] - a) < 2e-5
    sig = 1.0 / (1.0 + math.exp(-a))
    assert abs(sig * (1.0 + a * (1.0 - sig))) < 1e-14
    assert oracle.silu(a) <= sg.min() and sg.min() - oracle.silu(a) < 1e-10
    rng = np.random.default_rng(5)
    lo = rng.uniform(-6, 4, 300)
    hi = lo + rng.uniform(0, 3, 300)
    vmin, vmax = fp8.silu_range(lo, hi)
    for i in range(300):
        v = oracle.silu(np.linspace(lo[i], hi[i], 20001))
        assert vmin[i] <= v.min() + 1e-15 and v.min() - vmin[i] < 1e-8
        assert vmax[i] >= v.max() - 1e-15 and vmax[i] - v.max() < 1e-15


def test_activation_interval_holds_every_perturbed_accumulation():
    """Brute force: pre-activations moved anywhere inside acc_rel x their sums
    of |terms| (corners, random interior points) give SwiGLU values inside
    [h_lo, h_hi]; the interval is no wider than those moves reach (its ends
    are attained up to the fp32-evaluation slack); acc_rel = 0 leaves only
    the slack; the centre value is the exact activation."""
    rng = np.random.default_rng(8)
    R, d, I = 24, 256, 128
    u = rng.standard_normal((R, d))
    W1 = rng.standard_normal((I, d)) / 16
    W3 = rng.standard_normal((I, d)) / 16
    acc = 2.0 ** -6
    h, lo, hi = fp8.activation_interval(u, W1, W3, acc)
    a1, a3 = u @ W1.T, u @ W3.T
    np.testing.assert_array_equal(h, oracle.silu(a1) * a3)
    m1 = np.abs(u) @ np.abs(W1).T
    m3 = np.abs(u) @ np.abs(W3).T
    reach_lo, reach_hi = np.full_like(h, np.inf), np.full_like(h, -np.inf)
    moves = [(s1, s3) for s1 in (-1.0, 1.0) for s3 in (-1.0, 1.0)]
    moves += [(rng.uniform(-1, 1, h.shape), rng.uniform(-1, 1, h.shape)) for _ in range(200)]
    # the point where silu is smallest, wherever the a1 range contains it
    inside = np.abs(fp8.SILU_ARGMIN - a1) <= acc * m1
    t_min = np.where(inside, (fp8.SILU_ARGMIN - a1) / np.maximum(acc * m1, 1e-300), 1.0)
    moves += [(t_min, s3) for s3 in (-1.0, 1.0)]
    for e1, e3 in moves:
        hp = oracle.silu(a1 + e1 * acc * m1) * (a3 + e3 * acc * m3)
        assert np.all(hp >= lo) and np.all(hp <= hi)
        reach_lo, reach_hi = np.minimum(reach_lo, hp), np.maximum(reach_hi, hp)
    slack = 2.0 ** -20 * np.maximum(np.abs(lo), np.abs(hi))
    assert np.all(reach_lo - lo <= 1.0001 * slack + 1e-15)
    assert np.all(hi - reach_hi <= 1.0001 * slack + 1e-15)
    _, lo0, hi0 = fp8.activation_interval(u, W1, W3, 0.0)
    assert np.all(hi0 - lo0 <= 2.0 ** -19 * np.abs(h) * 1.0001 + 1e-300)


def test_admissible_codes():
    """The oracle's own quantisation of a value inside its interval is
    admissible; so is the quantisation of any other value inside it; a code two
    steps outside, a scale the group cannot have, and a flipped sign are
    not; a group whose intervals allow zero may take the zero group's scale."""
    rng = np.random.default_rng(9)
    h = rng.standard_normal((8, 256)) * np.exp(rng.uniform(-5, 5, (8, 1)))
    width = 1e-3 * np.abs(h) + 1e-6 * np.abs(h).max(axis=1, keepdims=True)
    lo, hi = h - width, h + width
    codes, scales = fp8.quantize_1x128(h)
    ok, sok = fp8.admissible_1x128(lo, hi, codes, scales)
    assert ok.all() and sok.all()
    for _ in range(20):
        inner = h + rng.uniform(-1, 1, h.shape) * width
        c2, s2 = fp8.quantize_1x128(inner)
        assert fp8.admissible_1x128(lo, hi, c2, s2)[0].all()
    # two code steps away from both interval ends (same sign, magnitude
    # below the largest code), for values well inside a code interval
    mag = codes & 0x7F
    movable = (mag >= 8) & (mag <= 0x7C)
    bumped = np.where(movable, codes + 2, codes).astype(np.uint8)
    bad, _ = fp8.admissible_1x128(lo, hi, bumped, scales)
    assert not bad[movable].any() and bad[~movable].all()
    wrong_scale = scales.copy()
    wrong_scale[0, 0] += 3
    ok2, sok2 = fp8.admissible_1x128(lo, hi, codes, wrong_scale)
    assert not sok2[0, 0] and not ok2[0, :128].any() and ok2[0, 128:].all()
    flipped = codes.copy()
    big = np.argmax(np.abs(h[1]))
    flipped[1, big] ^= 0x80
    assert not fp8.admissible_1x128(lo, hi, flipped, scales)[0][1, big]
    # intervals around zero: the all-zero group's scale byte (127) is allowed
    z_lo, z_hi = -np.full((1, 128), 1e-9), np.full((1, 128), 1e-9)
    zc = np.zeros((1, 128), np.uint8)
    assert fp8.admissible_1x128(z_lo, z_hi, zc, np.array([[127]], np.uint8))[0].all()


def test_forced_activations_reproduce_the_layer():
    """moe_forward_fp8 evaluated on its own quantised activations (given as
    forced_h) equals the plain evaluation; on other codes it follows them."""
    rng = np.random.default_rng(10)
    T, d, E, I, K = 48, 256, 6, 128, 2
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) / 16
    w1, w3 = (rng.standard_normal((E, I, d)) / 16 for _ in range(2))
    w2 = rng.standard_normal((E, d, I)) / 11
    s1, s3 = (rng.standard_normal((1, 128, d)) / 16 for _ in range(2))
    s2 = rng.standard_normal((1, d, 128)) / 11
    rq, sq = fp8.quantize_experts(w1, w3, w2), fp8.quantize_experts(s1, s3, s2)
    y, r = fp8.moe_forward_fp8(x, wg, rq, sq, K, n_shared=1)
    xd = _requant(x)

    def h_of(q, e, rows):
        W1 = fp8.dequantize_blocks(q[0][0][e], q[0][1][e])
        W3 = fp8.dequantize_blocks(q[1][0][e], q[1][1][e])
        return _requant(oracle.silu(rows @ W1.T) * (rows @ W3.T))
    hs = [h_of(sq, 0, xd)]
    hr = np.zeros((T, K, I))
    for e in np.unique(r.idx):
        tt, kk = np.nonzero(r.idx == e)
        hr[tt, kk] = h_of(rq, e, xd[tt])
    y2, _ = fp8.moe_forward_fp8(x, wg, rq, sq, K, n_shared=1, forced_h=(hs, hr))
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-13)
    hr2 = hr.copy()
    hr2[3, 1] *= 2.0
    y3, _ = fp8.moe_forward_fp8(x, wg, rq, sq, K, n_shared=1, forced_h=(hs, hr2))
    W2 = fp8.dequantize_blocks(rq[2][0][r.idx[3, 1]], rq[2][1][r.idx[3, 1]])
    np.testing.assert_allclose(y3[3] - y[3], r.g[3, 1] * (hr[3, 1] @ W2.T), rtol=1e-10,
                               atol=1e-12)
    assert np.array_equal(np.delete(y3, 3, 0), np.delete(y, 3, 0))
