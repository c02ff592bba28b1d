"""Pins for the oracle's number formats (E2M1 rounding, E8M0 exponent, packing).

Every expected value here comes from the format definitions (OCP Microscaling
v1.0: E2M1 = {0, 0.5, 1, 1.5, 2, 3, 4, 6} with sign, round to nearest, ties to
even, saturating; E8M0 shared exponent floor(log2 amax) - 2), computed by an
independent method: exact rational arithmetic over the whole grid.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import sharq_oracle as O

GRID_Q = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
          Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def brute_e2m1(t: float) -> int:
    """Nearest grid magnitude by exact distance to all eight points; on equal
    distance the even code wins; sign bit from t."""
    a = abs(Fraction(t))
    dists = [abs(a - g) for g in GRID_Q]
    best = min(dists)
    cands = [i for i, d in enumerate(dists) if d == best]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    sign = 1 if np.signbit(np.float64(t)) else 0
    return code | (sign << 3)


def _f32_neighbours(x: float, n: int) -> np.ndarray:
    b = np.array([x], dtype=np.float32).view(np.int32)[0]
    return (np.arange(b - n, b + n + 1, dtype=np.int64).astype(np.int32)).view(np.float32)


def test_e2m1_threshold_values():
    # closed-form decision points from the rounding rule
    cases = {0.0: 0, 0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7, 7.0: 7,
             7.99: 7, 1e30: 7}
    for t, code in cases.items():
        assert O.e2m1_nearest(np.float32(t)) == code, t
        assert O.e2m1_nearest(np.float32(-t)) == code | 8, -t
    nxt = np.nextafter(np.float32(0.25), np.float32(1))
    assert O.e2m1_nearest(nxt) == 1
    assert O.e2m1_nearest(np.nextafter(np.float32(5.0), np.float32(9))) == 7
    assert O.e2m1_nearest(np.float32(-0.0)) == 8


def test_e2m1_against_exact_bruteforce():
    vals = []
    # every finite bf16 value (upper half of binary32)
    b = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    f = b.view(np.float32)
    vals.append(f[np.isfinite(f)])
    # binary32 neighbourhoods of every midpoint and grid point
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 8.0]
    for p in pts:
        vals.append(_f32_neighbours(p, 40))
        vals.append(-_f32_neighbours(p, 40))
    # random binary32 in [-9, 9] and tiny/subnormal magnitudes
    rng = np.random.default_rng(1)
    vals.append(rng.uniform(-9, 9, 20000).astype(np.float32))
    vals.append(rng.integers(1, 1 << 23, 500).astype(np.uint32).view(np.float32))
    allv = np.concatenate(vals).astype(np.float32)
    got = O.e2m1_nearest(allv)
    # exact rational reference on a strided subset (all of it for the non-bf16 parts)
    sub = np.concatenate([allv[::7], allv[len(vals[0]):]])
    got_sub = O.e2m1_nearest(sub)
    want = np.array([brute_e2m1(float(t)) for t in sub], dtype=np.uint8)
    bad = np.nonzero(got_sub != want)[0]
    assert bad.size == 0, [(float(sub[i]), int(got_sub[i]), int(want[i])) for i in bad[:10]]
    # rounding is monotone in |t| and odd-symmetric
    pos = np.sort(np.abs(allv))
    c = O.e2m1_nearest(pos)
    assert np.all(np.diff(c.astype(np.int32)) >= 0)
    assert np.all(got & 7 == O.e2m1_nearest(np.abs(allv)))


@pytest.mark.slow
def test_e2m1_exhaustive_over_binary32():
    """Every non-negative finite binary32 value (2^31 - 2^23 bit patterns, about
    80 s).  The exact-rational rule is monotone in the bit pattern of a
    non-negative value, so its seven code boundaries -- the first pattern at or
    above each code -- are found by bisection with brute_e2m1, and the expected
    code of every pattern is the number of boundaries at or below it.  The
    oracle's code must equal it for all of them; the sign bit adds 8 (checked
    on every 64th pattern, and at -0)."""
    bounds = []
    for code in range(1, 8):
        lo, hi = 0, 0x7F800000
        while lo < hi:
            mid = (lo + hi) // 2
            if brute_e2m1(float(np.uint32(mid).view(np.float32))) >= code:
                hi = mid
            else:
                lo = mid + 1
        bounds.append(lo)
    bounds = np.array(bounds, dtype=np.uint64)
    chunk = 1 << 24
    for start in range(0, 0x7F800000, chunk):
        bits = np.arange(start, min(start + chunk, 0x7F800000), dtype=np.uint32)
        got = O.e2m1_nearest(bits.view(np.float32))
        want = np.searchsorted(bounds, bits.astype(np.uint64), side="right").astype(np.uint8)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"pattern {int(bits[bad[0]]):#010x}: {int(got[bad[0]])} != {int(want[bad[0]])}"
        neg = bits[::64] | np.uint32(0x80000000)
        assert np.array_equal(O.e2m1_nearest(neg.view(np.float32)), want[::64] | 8)
    assert O.e2m1_nearest(np.float32(np.inf)) == 7                # beyond the grid: saturates


def test_e2m1_value_roundtrip():
    for nib in range(16):
        v = O.e2m1_value(np.uint8(nib))
        assert O.e2m1_nearest(np.float32(v)) == nib


def test_floor_log2_exact():
    rng = np.random.default_rng(2)
    bits = rng.integers(1, 0x7F800000, 5000).astype(np.uint32)
    a = bits.view(np.float32)
    got = O.floor_log2(a)
    for x, g in zip(a[:600], got[:600]):
        q = Fraction(float(x))
        k = 0
        while Fraction(2) ** k > q:
            k -= 1
        while Fraction(2) ** (k + 1) <= q:
            k += 1
        assert g == k
    # subnormal and extreme ends
    assert O.floor_log2(np.float32(1.401298464324817e-45)) == -149
    assert O.floor_log2(np.float32(3.4028234663852886e38)) == 127


def test_e8m0_closed_forms():
    am = np.array([0.0, 1.0, 4.0, 6.0, 7.99, 8.0, 0.5, 2.0 ** -149, 3.4028234663852886e38,
                   2.0 ** -125, 2.0 ** -124], dtype=np.float32)
    e = O.mx_exponent(am)
    assert list(e + 127) == [0, 125, 127, 127, 127, 128, 124, 0, 252, 0, 1]


def test_mx_block_scale_invariant():
    rng = np.random.default_rng(3)
    u = (rng.standard_normal((200, 64)) * np.exp2(rng.integers(-30, 30, (200, 1)))).astype(np.float32)
    sc, nib = O.quantize_mx(u)
    e = sc.astype(np.int64) - 127
    amax = np.abs(u.reshape(200, 2, 32)).max(-1).astype(np.float64)
    ratio = amax / np.exp2(e)
    assert np.all((ratio >= 4) & (ratio < 8))
    # the block maximum lands on 4 or 6 (codes 6 / 7)
    blocks = nib.reshape(200, 2, 32) & 7
    idx = np.abs(u.reshape(200, 2, 32)).argmax(-1)
    top = np.take_along_axis(blocks, idx[..., None], -1)[..., 0]
    assert np.all((top == 6) | (top == 7))
    # dequantised error at most half a grid step (or the saturation gap 6..8)
    d = O.dequant_mx(sc, nib).reshape(200, 2, 32)
    t = u.reshape(200, 2, 32).astype(np.float64) / np.exp2(e)[..., None]
    q = d / np.exp2(e)[..., None]
    a = np.abs(t)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert np.all(np.abs(t - q) <= step / 2 + (a > 6) * 2)


def test_mx_closed_form_block():
    # block [6, 0.5, 1, ...] at scale 2^10: codes unchanged, E = 127 + 10
    base = np.array([6, 0.5, 1, -1.5, 2, -3, 4, 0] * 4, dtype=np.float32)
    for sh in (0, 10, -20):
        sc, nib = O.quantize_mx((base * np.float32(2.0 ** sh))[None])
        assert sc[0, 0] == 127 + sh
        assert list(nib[0, :8]) == [7, 1, 2, 11, 4, 13, 6, 0]
    # all-zero block -> E = 0, codes 0 (and -0 -> 0x8)
    z = np.zeros((1, 32), dtype=np.float32)
    z[0, 5] = -0.0
    sc, nib = O.quantize_mx(z)
    assert sc[0, 0] == 0 and nib[0, 5] == 8 and nib[0].sum() == 8


def test_nibble_and_meta_packing():
    nib = np.arange(16, dtype=np.uint8)[None]
    b = O.pack_nibbles(nib)
    assert list(b[0]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(O.unpack_nibbles(b), nib)
    kept = np.array([[1, 0, 1, 0, 0, 1, 0, 1]], dtype=bool)
    meta = O.pack_meta_24(kept)
    assert meta[0, 0] == (0 | 2 << 2) | ((1 | 3 << 2) << 4)
    assert np.array_equal(O.unpack_meta_24(meta, 8), kept)
    with pytest.raises(ValueError):
        O.pack_meta_24(np.ones((1, 8), dtype=bool))
