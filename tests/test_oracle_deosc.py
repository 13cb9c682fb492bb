"""Pins of the oracle's weight de-oscillation (hysteresis on the 32x32 weight
quantizer) against what its definition fixes.

The reading ("AMD's ALTO Gets 4-Bit MoE Training to Within 0.007 of BF16",
section "What ALTO Actually Does": a master weight near a rounding boundary
flips between two levels under tiny updates; the recipe damps this with a
simplified de-oscillation step): while a tile's scale is unchanged, an
element keeps its previous level until its scaled value leaves that level's
rounding interval widened by margin/64 of a grid step on each side.

- hand-worked threshold cases (values on, inside and outside the band);
- margin 0 changes no decoded value against plain round-to-nearest-even;
- quantizing a tensor against its own quantization keeps every code;
- a changed tile scale disables the band;
- flip counts equal a brute-force count of changed decoded values;
- the kept set grows with the margin; transposition commutes with the rule;
- on a random-walk master-weight trajectory the flips per step fall as the
  margin grows.
"""
import numpy as np
import pytest

import oracle

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _tile_with(value, amax=4.0):
    """A 1x32x32 fp32 tile: element (0, 0) = amax (scale 2^0 for amax in
    [4, 8)), element (1, 1) = value, the rest 0."""
    w = np.zeros((1, 32, 32), dtype=np.float32)
    w[0, 0, 0] = amax
    w[0, 1, 1] = value
    return w


def _prev_with(code, scale_byte=127):
    """Previous state: every element code 0 except (0, 0) = +4 (code 6) and
    (1, 1) = `code`; one scale byte."""
    c = np.zeros((1, 32, 16), dtype=np.uint8)
    c[0, 0, 0] = 0x06
    c[0, 1, 0] = np.uint8(code << 4)          # element (1, 1): high nibble of byte (1, 0)
    s = np.full((1, 1, 1), scale_byte, dtype=np.uint8)
    return c, s


def _code_at_11(codes):
    return int(codes[0, 1, 0] >> 4)


# (previous code, margin64, scaled value, expected code), worked by hand from
# the definition: band = (q - f (q - q_dn), q + f (q_up - q)), f = 1/2 + m/64
HAND = [
    # prev +1.0, f = 0.625: neighbours 0.5 and 1.5 -> band (0.6875, 1.3125)
    (0x2, 8, 1.3, 0x2),        # RTNE would give 1.5
    (0x2, 8, 1.3125, 0x3),     # on the band's edge: not inside -> RTNE 1.5
    (0x2, 8, 0.69, 0x2),       # RTNE would give 0.5
    (0x2, 8, 0.6875, 0x1),     # edge -> RTNE 0.5
    (0x2, 0, 1.26, 0x3),       # margin 0: the plain rounding interval
    (0x2, 31, 1.49, 0x2),      # f = 63/64: band up to 1.4921875
    (0x2, 31, 1.4921875, 0x3),
    # prev -0 (code 8): neighbours -0.5 and +0.5, f = 0.625 -> (-0.3125, 0.3125)
    (0x8, 8, 0.3, 0x8),        # RTNE would give +0.5; the kept code keeps its sign
    (0x8, 8, 0.3125, 0x1),
    (0x0, 8, -0.3, 0x0),
    # prev +6 (code 7): neighbour 4 below, open above: band (4.75, inf)
    (0x7, 8, 4.8, 0x7),        # RTNE would give 4
    (0x7, 8, 4.75, 0x6),
    (0x7, 8, 7.9, 0x7),
    # prev -6 with a positive value: far outside -> RTNE (5.0 is a tie -> 4)
    (0xF, 8, 5.0, 0x6),
    # prev +0.5: band (0.1875, 0.8125); a negative value leaves it
    (0x1, 8, -0.1, 0x8),
    (0x1, 8, 0.19, 0x1),
    (0x1, 8, 0.8, 0x1),
    (0x1, 8, 0.8125, 0x2),
    # prev -3 (code D): neighbours -4 and -2, f = 0.75 -> (-3.75, -2.25)
    (0xD, 16, -3.7, 0xD),
    (0xD, 16, -2.5, 0xD),      # RTNE would give -2 (tie to even)
    (0xD, 16, -2.26, 0xD),
    (0xD, 16, -2.25, 0xC),     # edge -> RTNE(-2.25) = -2
    (0xD, 16, -3.75, 0xE),     # edge -> RTNE(-3.75) = -4
]


@pytest.mark.parametrize("prev,margin,v,want", HAND)
def test_hand_worked_band_edges(prev, margin, v, want):
    w = _tile_with(v)
    pc, ps = _prev_with(prev)
    codes, scales, _, _, _ = oracle.quantize_2d_deosc(w, pc, ps, margin)
    assert int(scales[0, 0, 0]) == 127
    assert _code_at_11(codes) == want, (hex(prev), margin, v, hex(_code_at_11(codes)))


def _random_weights(seed, batch=2, rows=64, cols=96):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((batch, rows, cols)) * 0.02).astype(np.float32)


def _values(codes, scales):
    b, r, h = codes.shape
    return np.stack([oracle.dequantize(codes[k], scales[k], block_rows=32) for k in range(b)])


def test_margin_zero_changes_no_value():
    w = _random_weights(1)
    prev = oracle.quantize_2d(_random_weights(2) * 0.5 + w)
    plain = oracle.quantize_2d(w)
    got = oracle.quantize_2d_deosc(w, prev[0], prev[1], 0)
    assert np.array_equal(got[1], plain[1])
    assert np.array_equal(_values(got[0], got[1]), _values(plain[0], plain[1]))


def test_own_quantization_keeps_every_code():
    w = _random_weights(3)
    c, s, ct, st = oracle.quantize_2d(w)
    for m in (0, 8, 31):
        got = oracle.quantize_2d_deosc(w, c, s, m)
        assert np.array_equal(got[0], c) and np.array_equal(got[2], ct)
        assert np.array_equal(got[1], s) and np.array_equal(got[3], st)
        assert not got[4].any()


def test_changed_scale_disables_the_band():
    # previous scale byte 126 (the tile's rule gives 127): plain RTNE
    w = _tile_with(1.3)
    pc, ps = _prev_with(0x2, scale_byte=126)
    codes, scales, _, _, flips = oracle.quantize_2d_deosc(w, pc, ps, 31)
    assert _code_at_11(codes) == 0x3
    assert np.array_equal(codes, oracle.quantize_2d(w)[0])
    assert int(flips[0, 0, 0]) == 2        # both nonzero elements change value (2^-1 scale step)


def test_flip_counts_by_brute_force():
    rng = np.random.default_rng(5)
    w0 = _random_weights(6, batch=3)
    prev = oracle.quantize_2d(w0)
    w1 = w0 + (rng.standard_normal(w0.shape) * 3e-3).astype(np.float32)
    w1[0, :32, :32] *= 3.0                  # one tile changes its scale
    w1[1, 32:, 64:] = np.nan                # one tile becomes non-finite
    for m in (0, 12):
        c, s, _, _, flips = oracle.quantize_2d_deosc(w1, prev[0], prev[1], m)
        before, now = _values(prev[0], prev[1]), _values(c, s)
        changed = ~(before == now)           # NaN on either side counts
        want = changed.reshape(3, 2, 32, 3, 32).sum(axis=(2, 4))
        assert np.array_equal(flips.astype(np.int64), want)


def test_each_code_is_the_previous_or_the_rtne_code_and_kept_sets_grow():
    rng = np.random.default_rng(7)
    w0 = _random_weights(8, batch=2, rows=96, cols=128)
    prev = oracle.quantize_2d(w0)
    w1 = w0 + (rng.standard_normal(w0.shape) * 2e-3).astype(np.float32)
    plain = oracle.quantize_2d(w1)[0]

    def nib(c):
        return np.stack([c & 0xF, c >> 4], axis=-1)

    kept_before = None
    for m in (0, 4, 12, 24, 31):
        c = oracle.quantize_2d_deosc(w1, prev[0], prev[1], m)[0]
        n, p, r = nib(c), nib(prev[0]), nib(plain)
        assert np.all((n == p) | (n == r))
        kept = (n == p) & (p != r)
        if kept_before is not None:
            assert np.all(kept[kept_before]), m
        kept_before = kept
    assert kept_before.sum() > 0


def test_transpose_commutes_with_the_rule():
    rng = np.random.default_rng(9)
    w0 = _random_weights(10, batch=1, rows=64, cols=128)
    w1 = w0 + (rng.standard_normal(w0.shape) * 2e-3).astype(np.float32)
    prev = oracle.quantize_2d(w0)
    a = oracle.quantize_2d_deosc(w1, prev[0], prev[1], 16)
    wt = np.ascontiguousarray(np.swapaxes(w1, 1, 2))
    b = oracle.quantize_2d_deosc(wt, prev[2], prev[3], 16)
    assert np.array_equal(a[2], b[0]) and np.array_equal(a[3], b[1])
    assert np.array_equal(a[0], b[2]) and np.array_equal(a[1], b[3])
    assert np.array_equal(a[4], np.swapaxes(b[4], 1, 2))


def test_random_walk_flips_fall_with_the_margin():
    """Master weights N(0, 0.02) take 30 steps of a zero-mean random walk of
    1e-4 per step (updates near 1% of a level step): with margin 0 a few
    weights near a boundary flip every step; the band removes most flips."""
    rng = np.random.default_rng(11)
    w = _random_weights(12, batch=4, rows=64, cols=64)
    steps = [(rng.standard_normal(w.shape) * 1e-4).astype(np.float32) for _ in range(30)]
    totals = {}
    for m in (0, 4, 16):
        cur = w.copy()
        c, s, _, _ = oracle.quantize_2d(cur)
        tot = 0
        for d in steps:
            cur = cur + d
            c, s, _, _, flips = oracle.quantize_2d_deosc(cur, c, s, m)
            tot += int(flips.sum())
        totals[m] = tot
    assert totals[0] > 0
    assert totals[0] > totals[4] > totals[16], totals
    assert totals[16] * 5 < totals[0], totals


# (previous byte, margin64, tile amax, expected byte): the scale band keeps
# the previous byte p when the rule gives p - 1 and amax >= (4 - m/16) 2^(p-127)
SCALE_HAND = [
    (127, 8, 3.9, 127),     # rule 126; 3.9 >= 3.5: kept
    (127, 8, 3.5, 127),     # on the threshold: kept (>=)
    (127, 8, 3.49, 126),    # below it
    (127, 0, 3.99, 126),    # margin 0: no scale band
    (127, 31, 2.0625, 127),  # the widest band: 4 - 31/16
    (127, 31, 2.06, 126),
    (126, 8, 4.5, 127),     # upward: never held back
    (128, 31, 3.9, 126),    # two binades down: not held
    (0xFF, 31, 3.9, 126),   # no previous scale
]


@pytest.mark.parametrize("pbyte,margin,amax,want", SCALE_HAND)
def test_hand_worked_scale_band(pbyte, margin, amax, want):
    w = _tile_with(0.3, amax=amax)
    pc, ps = _prev_with(0x1, scale_byte=pbyte)
    codes, scales, _, _, _ = oracle.quantize_2d_deosc(w, pc, ps, margin)
    assert int(scales[0, 0, 0]) == want
    # the tile's amax element, at the kept or the new scale: RTNE there
    big = int(codes[0, 0, 0]) & 0xF
    X = want - 127
    assert GRID[big & 7] == GRID[oracle.rtne_mag(amax / 2.0 ** X)]


def test_scale_band_improves_the_largest_value():
    """amax 3.9 at a previous scale 2^0: the plain rule (2^-1) saturates it
    to 6 * 2^-1 = 3 (error 0.9); the kept scale represents it as 4 (0.1)."""
    w = _tile_with(0.3, amax=3.9)
    pc, ps = _prev_with(0x1, scale_byte=127)
    kept = oracle.quantize_2d_deosc(w, pc, ps, 8)
    plain = oracle.quantize_2d(w)
    assert oracle.dequantize(kept[0][0], kept[1][0], block_rows=32)[0, 0] == 4.0
    assert oracle.dequantize(plain[0][0], plain[1][0], block_rows=32)[0, 0] == 3.0


def test_amax_hovering_at_a_power_of_two_stops_flipping():
    """A tile whose largest weight alternates 4.01 / 3.99 (times 2^-5) while
    the rest stay put: without the band every element's value changes at
    each crossing; with it, after the first step nothing changes."""
    rng = np.random.default_rng(13)
    base = (rng.standard_normal((1, 32, 32)) * 0.02).astype(np.float32)
    base[0, 5, 7] = 4.01 * 2.0 ** -5
    c, s, _, _ = oracle.quantize_2d(base)
    totals = {}
    for m in (0, 8):
        cc, ss, tot = c, s, 0
        for k in range(8):
            w = base.copy()
            w[0, 5, 7] = (3.99 if k % 2 == 0 else 4.01) * 2.0 ** -5
            cc, ss, _, _, fl = oracle.quantize_2d_deosc(w, cc, ss, m)
            tot += int(fl.sum())
        totals[m] = tot
    assert totals[0] > 8 * 300, totals       # hundreds of values move at every crossing
    assert totals[8] == 0, totals
