"""Pins of the dynamic tree codebook of the oracle codec.

The abstract of "4-bit Shampoo for Memory-Efficient Network Training" compares its
linear-square codebook with dynamic tree quantization, whose definition is not on the
pages (they cite the 8-bit optimizers paper that defines it by title only).  The levels
are pinned here against the published bit-level rule worked out by hand, the codec
mechanics against brute force, and the whole step against the diagonal special case
(all CPU).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import ablation as ab
from oracle import codec
from oracle import shampoo4 as o
from workloads import get_workload

DT = codec.DYNAMIC_TREE


def test_levels_hand_worked():
    """Worked by hand from the rule: a 3-bit magnitude with E leading zeros keeps
    2 - E fraction bits, whose 2^(2-E) values are the midpoints of equal bins of
    [0.1, 1] scaled by 10^-E.
      E = 0 (patterns 1xx): bins of 0.225 -> 0.2125 0.4375 0.6625 0.8875
      E = 1 (patterns 01x): bins of 0.45, times 0.1 -> 0.0325 0.0775
      E = 2 (pattern 001): one bin, midpoint 0.55, times 0.01 -> 0.0055
      000 -> 0; sign bit with 000 -> +1 (the block maximum)."""
    pos = ["0.0055", "0.0325", "0.0775", "0.2125", "0.4375", "0.6625", "0.8875"]
    want = [-Fraction(v) for v in reversed(pos)] + [Fraction(0)] + [Fraction(v) for v in pos] + [Fraction(1)]
    assert codec.exact_levels_of(DT) == want
    assert np.array_equal(codec.levels(DT), np.array([float(v) for v in want], np.float32))


def test_bit_patterns_cover_the_codebook_once():
    vals = [codec.dynamic_tree_value(t) for t in range(16)]
    assert len(set(vals)) == 16
    lv = codec.exact_levels_of(DT)
    codes = [lv.index(v) for v in vals]
    assert sorted(codes) == list(range(16))
    assert codes[0] == codec.ZERO_CODE          # pattern 0000 is the zero level
    assert codes[8] == 15                       # pattern 1000 is +1
    for t in range(1, 8):                       # the sign bit negates every other value
        assert vals[t | 8] == -vals[t]


def test_decades_are_linear():
    """Inside each decade the levels are evenly spaced and centred in their bins."""
    lv = codec.exact_levels_of(DT)
    pos = [v for v in lv if 0 < v < 1]
    for e, count in ((0, 4), (1, 2), (2, 1)):
        lo, hi = Fraction(1, 10 ** (e + 1)), Fraction(1, 10 ** e)
        dec = [v for v in pos if lo < v < hi]
        assert len(dec) == count
        width = (hi - lo) / count
        assert dec == [lo + width * (k + Fraction(1, 2)) for k in range(count)]


def _codes_for_xhat(xhat):
    """Quantize values x_hat in [-1, 1] with block scale 1 (each block starts with 1.0)."""
    per = 63
    n = xhat.size
    nb = (n + per - 1) // per
    blocks = np.zeros((nb, 64), np.float32)
    blocks[:, 0] = 1.0
    flat = np.zeros(nb * per, np.float32)
    flat[:n] = xhat
    blocks[:, 1:] = flat.reshape(nb, per)
    c, s = codec.quantize(blocks.ravel(), 64, DT)
    assert np.all(s == 1.0)
    return codec.unpack_nibbles(c).reshape(nb, 64)[:, 1:].ravel()[:n]


def test_quantize_matches_bruteforce_nearest_level():
    """Codes are the exact nearest level (ties to the lower code) except inside the
    float32 rounding interval of a midpoint."""
    rng = np.random.default_rng(31)
    mids32 = codec.midpoints(DT)
    samples = [rng.uniform(-1, 1, 3000).astype(np.float32),
               (rng.uniform(-1, 1, 2000) ** 3).astype(np.float32)]   # dense near zero
    for m in mids32:
        around = [m]
        up = down = np.float32(m)
        for _ in range(30):
            up = np.nextafter(up, np.float32(2))
            down = np.nextafter(down, np.float32(-2))
            around += [up, down]
        samples.append(np.array(around, np.float32))
    samples.append(np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40], np.float32))
    xs = np.concatenate(samples)
    got = _codes_for_xhat(xs)
    lv = codec.exact_levels_of(DT)
    exact_mids = [(lv[j] + lv[j + 1]) / 2 for j in range(15)]
    for x, c in zip(xs.tolist(), got.tolist()):
        fx = Fraction(x)
        dist = [abs(fx - q) for q in lv]
        e = dist.index(min(dist))
        if c == e:
            continue
        j = min(c, e)
        assert abs(c - e) == 1
        a, b = sorted([Fraction(float(mids32[j])), exact_mids[j]])
        assert a <= fx <= b, (x, c, e)


def test_ties_go_to_lower_code():
    m = codec.midpoints(DT)
    assert _codes_for_xhat(m).tolist() == list(range(15))
    assert _codes_for_xhat(np.nextafter(m, np.float32(2))).tolist() == list(range(1, 16))


def test_round_trip_exact_on_codebook_values():
    rng = np.random.default_rng(32)
    lv = codec.levels(DT)
    for _ in range(40):
        s = np.float32(10.0 ** rng.uniform(-6, 3))
        codes = rng.integers(0, 16, 64)
        codes[rng.integers(0, 64)] = 15                 # +1: the absmax level
        x = (lv[codes] * s).astype(np.float32)
        c, sc = codec.quantize(x, 64, DT)
        assert sc[0] == s
        assert codec.unpack_nibbles(c).tolist() == codes.tolist()
        assert np.array_equal(codec.dequantize(c, sc, 64, 64, DT).view(np.uint32), x.view(np.uint32))


def test_negative_block_maximum_is_not_exact():
    """Only +1 is a level: a block whose absmax element is negative loses it to -0.8875."""
    x = np.zeros(64, np.float32)
    x[0], x[1] = -2.0, 1.0
    c, s = codec.quantize(x, 64, DT)
    y = codec.dequantize(c, s, 64, 64, DT)
    assert s[0] == 2.0 and y[0] == np.float32(-0.8875) * np.float32(2.0) and y[1] == np.float32(0.4375 * 2)


@pytest.mark.parametrize("p", [1, 3, 33, 64, 100])
def test_identity_is_exact(p):
    c, s = codec.quantize_matrix(np.eye(p, dtype=np.float32), 64, DT)
    assert np.array_equal(codec.dequantize_matrix(c, s, p, 64, DT), np.eye(p, dtype=np.float32))


def test_diagonal_gradients_reduce_to_rmsprop():
    """With either codebook U stays I under diagonal gradients, so the step is RMSprop."""
    rng = np.random.default_rng(33)
    p, beta, eps = 12, 0.9, 1e-6
    orc = o.Shampoo4Oracle([(p, p)], beta=beta, eps=eps, codebook=DT)
    v = np.zeros(p, np.float32)
    b32 = np.float32(beta)
    for t in range(1, 6):
        g = rng.standard_normal(p).astype(np.float32)
        P = orc.step([np.diag(g)], t)[0]
        v = (np.float64(b32) * v + (1.0 - np.float64(b32)) * g.astype(np.float64) ** 2).astype(np.float32)
        assert np.allclose(np.diag(P), g / np.sqrt(v.astype(np.float64) + float(np.float32(eps))),
                           rtol=1e-6, atol=1e-30)


def test_linear_square_beats_dynamic_tree():
    """The abstract's comparison on the workloads' own statistics: 4-bit eigenvectors
    coded with linear-square give a more accurate inverse root than with dynamic tree,
    with and without rectification."""
    for name in ("single_64x32", "cnn_batch"):
        wl = get_workload(name)
        L = ab.ema_factor([wl.block_gradient(0, t) for t in range(1, 11)], wl.beta)
        truth = ab.inverse_root(L, 1e-6)
        for k in (0, 1):
            ls = ab.rel_err(ab.root_eigvec4(L, 1e-6, k, codebook=codec.LINEAR_SQUARE), truth)
            dt = ab.rel_err(ab.root_eigvec4(L, 1e-6, k, codebook=DT), truth)
            assert ls < dt, (name, k, ls, dt)
