"""Pins for the oracle's NVFP4-style format (a reading: the SharQ abstract names
NVFP4 without defining it; the oracle follows the public two-level NVFP4
description -- E2M1 elements, OCP E4M3 scale per 16 elements, binary32 scale
per tensor, g = amax / (6 * 448)).

The expected values come from the definitions by independent routes: E4M3
decoded from its bit fields with exact rationals, round-to-nearest-even by
brute force over the whole E4M3 grid, correctly rounded binary32 of exact
rational quotients, and element codes by exact distance to the E2M1 grid.
"""
from fractions import Fraction

import numpy as np
import pytest

from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O

E2M1_Q = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
          Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_exact(byte: int) -> Fraction:
    """OCP E4M3 (sign clear): exponent field e (bias 7), mantissa m; e == 0 is
    subnormal with exponent 1 - 7."""
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(2) ** -6
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


GRID = [e4m3_exact(b) for b in range(127)]          # 0x7F is NaN
GRID_F = np.array([float(g) for g in GRID])


def rn32(q: Fraction) -> np.float32:
    """Correctly rounded binary32 of a positive or zero rational (ties to even)."""
    if q == 0:
        return np.float32(0.0)
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0))]
    best = min(abs(Fraction(float(c)) - q) for c in cands)
    near = [c for c in cands if abs(Fraction(float(c)) - q) == best]
    if len(near) == 1:
        return near[0]
    return [c for c in near if int(np.array(c).view(np.uint32)) % 2 == 0][0]


def brute_e4m3_byte(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value by exact float64 distance to all 127 values (exact for
    binary32 x in [0, 2^11]); equal distances go to the even byte."""
    d = np.abs(x.astype(np.float64)[:, None] - GRID_F[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(cand.sum(1) == 1, cand.argmax(1), even.argmax(1))
    return pick.astype(np.uint8)


def brute_e2m1(q: Fraction, negative: bool) -> int:
    a = abs(q)
    dists = [abs(a - g) for g in E2M1_Q]
    best = min(dists)
    cands = [i for i, dd in enumerate(dists) if dd == best]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return code | (8 if negative else 0)


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_and_roundtrip():
    vals = O.e4m3_value(np.arange(127))
    assert [Fraction(float(v)) for v in vals] == GRID
    assert np.all(np.diff(vals) > 0)                   # strictly increasing in the byte
    assert vals[-1] == 448.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    v, b = O.e4m3_round(vals.astype(np.float32))
    assert np.array_equal(b, np.arange(127, dtype=np.uint8)) and np.array_equal(v, vals)


@pytest.mark.slow
def test_e4m3_exhaustive_over_binary32():
    """Every binary32 value in [2^-11, 480] (about 1.7e8 patterns, where all the
    rounding decisions lie), and every 4096th pattern from 0 to 2^-11 and from
    480 to the largest finite value.  The nearest-value rule is monotone in the
    bit pattern, so the first pattern at or above each byte is found by
    bisection with brute_e4m3_byte, and the expected byte of every pattern is
    the number of those boundaries at or below it (bytes 0..126 increase with
    their values)."""
    bounds = []
    top = int(np.float32(2.0 ** 11).view(np.uint32))               # the brute force is exact up to 2^11
    for byte in range(1, 127):
        lo, hi = 0, top
        while lo < hi:
            mid = (lo + hi) // 2
            if brute_e4m3_byte(np.array([np.uint32(mid)]).view(np.float32))[0] >= byte:
                hi = mid
            else:
                lo = mid + 1
        bounds.append(lo)
    bounds = np.array(bounds, dtype=np.uint64)
    lo_bits = int(np.float32(2.0 ** -11).view(np.uint32))
    hi_bits = int(np.float32(480.0).view(np.uint32))
    assert bounds[0] > lo_bits and bounds[-1] <= hi_bits          # every decision inside the dense range
    ranges = [np.arange(0, lo_bits, 4096, dtype=np.uint32),
              np.arange(hi_bits, 0x7F800000, 4096, dtype=np.uint32)]
    chunk = 1 << 24
    ranges += [np.arange(s0, min(s0 + chunk, hi_bits), dtype=np.uint32) for s0 in range(lo_bits, hi_bits, chunk)]
    for bits in ranges:
        v, b = O.e4m3_round(bits.view(np.float32))
        want = np.searchsorted(bounds, bits.astype(np.uint64), side="right").astype(np.uint8)
        bad = np.nonzero(b != want)[0]
        assert bad.size == 0, f"pattern {int(bits[bad[0]]):#010x}: byte {int(b[bad[0]])} != {int(want[bad[0]])}"
        assert np.array_equal(v, GRID_F[want])


def test_e4m3_round_against_bruteforce():
    pts = []
    f = GRID_F
    mids = 0.5 * (f[:-1] + f[1:])
    for p in np.concatenate([mids, f[1:]]):
        b = np.array([p], dtype=np.float32).view(np.int32)[0]
        pts.append((np.arange(b - 30, b + 31).astype(np.int32)).view(np.float32))
    rng = np.random.default_rng(3)
    pts.append(np.exp2(rng.uniform(-14, 10.9, 40000)).astype(np.float32))
    pts.append(np.array([0.0, 2.0 ** -10, 3 * 2.0 ** -11, 464.0, 480.0, 2047.0], dtype=np.float32))
    x = np.concatenate(pts)
    x = x[(x >= 0) & (x <= 2048)]
    v, b = O.e4m3_round(x)
    want = brute_e4m3_byte(x)
    bad = np.nonzero(b != want)[0]
    assert bad.size == 0, [(float(x[i]), int(b[i]), int(want[i])) for i in bad[:8]]
    assert np.array_equal(v, GRID_F[want])
    # saturation: everything above 448 maps to 448 (no infinity / NaN code)
    big = np.array([448.0, 449.0, 464.0, 479.0, 480.0, 1e6, 3e38], dtype=np.float32)
    vb, bb = O.e4m3_round(big)
    assert np.all(vb == 448.0) and np.all(bb == 126)


def test_tensor_scale_closed_forms():
    assert O.nv_tensor_scale(2688.0) == 1.0
    assert O.nv_tensor_scale(1344.0) == 0.5
    assert O.nv_tensor_scale(0.0) == 1.0
    assert O.nv_tensor_scale(1.0) == rn32(Fraction(1, 2688))
    assert O.nv_tensor_scale(np.float32(3.7)) == rn32(Fraction(float(np.float32(3.7))) / 2688)


# ------------------------------------------------------------------ quantiser
def test_closed_form_blocks():
    """Hand-derived blocks with tensor scale g = 1 (tensor amax 2688).

    block 0: amax 2688 -> s = 448 -> t = 448; 2688/448 = 6 (code 7); 672/448 =
             1.5 (3); -224/448 = -0.5 (9); 112/448 = 0.25 (tie, even code 0).
    block 1: amax 12 -> s = 2 (byte 0x40); 12/2 = 6 (7); 3/2 = 1.5 (3);
             -1/2 = -0.5 (9); 0.5/2 = 0.25 (0); 2.5/2 = 1.25 (tie 1 | 1.5 -> 2);
             7/2 = 3.5 (tie 3 | 4 -> 6); -5/2 = -2.5 (tie 2 | 3 -> 4, sign: 12).
    block 2: all zero -> s = 0, codes 0 (and 8 for -0).
    block 3: amax 0.005 -> 0.005/6 < 2^-10 rounds to s = 0 -> signed zero codes.
    block 4: amax 0.006 -> 0.006/6 = 0.001 -> s = 2^-9 (byte 1); 0.006/2^-9 =
             3.072 (code 5); -0.0015/2^-9 = -0.768 (code 10).
    """
    blocks = np.zeros((5, 16), dtype=np.float32)
    blocks[0, :4] = [2688, 672, -224, 112]
    blocks[1, :7] = [12, 3, -1, 0.5, 2.5, 7, -5]
    blocks[2, 1] = -0.0
    blocks[3, :2] = [0.005, -0.001]
    blocks[4, :2] = [0.006, -0.0015]
    sc, nib = O.quantize_nv(blocks.reshape(1, 80), F := np.float32(1.0))
    nib = nib.reshape(5, 16)
    assert list(sc[0]) == [126, 0x40, 0, 0, 1]
    assert list(nib[0, :5]) == [7, 3, 9, 0, 0]
    assert list(nib[1, :8]) == [7, 3, 9, 0, 2, 6, 12, 0]
    assert nib[2, 1] == 8 and nib[2, 0] == 0
    assert list(nib[3, :3]) == [0, 8, 0]
    assert list(nib[4, :3]) == [5, 10, 0]
    d = O.dequant_nv(sc, nib.reshape(1, 80), F).reshape(5, 16)
    assert list(d[1, :7]) == [12, 3, -1, 0, 2, 8, -4]


def _check_codes(u, g, sc, nib):
    """Every block scale and element code from exact rationals."""
    u = np.asarray(u, dtype=np.float32)
    K = u.shape[-1]
    G = Fraction(float(g))
    for r in range(u.shape[0]):
        for b in range(K // 16):
            blk = u[r, 16 * b:16 * b + 16]
            amax = Fraction(float(np.abs(blk).max()))
            q = rn32(amax / Fraction(float(np.float32(6 * float(g)))))  # 6g: 26 bits, exact in float64
            sb = int(brute_e4m3_byte(np.array([q]))[0])
            assert sc[r, b] == sb, (r, b)
            t = rn32(e4m3_exact(sb) * G)
            for i, val in enumerate(blk):
                k = 16 * b + i
                neg = bool(np.signbit(val))
                if sb == 0:
                    assert nib[r, k] == (8 if neg else 0)
                    continue
                Q = Fraction(float(val)) / t
                want = brute_e2m1(Q, neg)
                if nib[r, k] != want:
                    # only a binary32 rounding of Q onto a decision point may move it
                    q32 = Fraction(float(rn32(abs(Q))))
                    assert q32 in (Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4),
                                   Fraction(5, 2), Fraction(7, 2), Fraction(5)), (r, k)


def test_quantize_nv_against_exact_rationals():
    rng = np.random.default_rng(11)
    u = (rng.standard_normal((3, 64)) * np.exp2(rng.integers(-6, 6, (3, 1)))).astype(np.float32)
    u[0, :16] *= 1e-4                                   # a block with a small scale
    g = O.nv_tensor_scale(np.abs(u).max())
    sc, nib = O.quantize_nv(u, g)
    _check_codes(u, g, sc, nib)


def test_block_max_code_invariant():
    """s rounds amax/(6g) by at most 1/16 relative in the normal E4M3 range, so
    each block's largest element lands on 6 (code 7).  A nonzero subnormal
    s is amax/(6g) rounded to a multiple of 2^-9, which lies in [2/3, 2) times
    it, so the largest quotient lies in (3, 9] and its code is 5, 6 or 7."""
    rng = np.random.default_rng(12)
    u = (rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-22, 0, (64, 16)).repeat(16, 1))).astype(np.float32)
    g = O.nv_tensor_scale(np.abs(u).max())
    sc, nib = O.quantize_nv(u, g)
    s = O.e4m3_value(sc)
    mag = (nib & 7).reshape(64, 16, 16).max(-1)
    assert np.all(mag[s >= 2.0 ** -6] == 7)
    sub = (s > 0) & (s < 2.0 ** -6)
    assert sub.any() and np.all(mag[sub] >= 5)
    assert np.all(mag[s == 0] == 0)


# ------------------------------------------------------------------ prepare
@pytest.mark.parametrize("name,M", [("decode1", 1), ("decode8", 8), ("qkv", 6)])
def test_prepare_nv_invariants(name, M):
    inp = synth.layer_inputs(name, seed=1, M=M, with_weight=False)
    out = O.prepare_nv(inp["x"], inp["gamma"], inp["eps"])
    v, d, r, kept = out["v"], out["d"], out["r"], out["kept"]
    K = v.shape[1]
    g = kept.reshape(M, K // 4, 4)
    assert np.all(g.sum(-1) == 2)
    # the residual subtraction is exact (d within a factor 2 of v wherever kept)
    assert np.array_equal(d.astype(np.float64) + r.astype(np.float64), v.astype(np.float64))
    assert np.array_equal(r[~kept].view(np.uint32), v[~kept].view(np.uint32))
    # tensor scales: the backbone keeps each group's maximum, so max|S| = max|v|
    assert out["g_s"] == rn32(Fraction(float(np.abs(v).max())) / 2688)
    assert out["g_r"] == rn32(Fraction(float(np.abs(r).max())) / 2688)
    assert np.array_equal(O.unpack_meta_24(out["s_meta"], K), kept)
    assert out["s_scales"].shape == (M, K // 16) == out["r_scales"].shape
    # every scale and code of both tensors from exact rationals, on a few rows
    rows = [0, M - 1]
    _check_codes(np.where(kept, v, 0)[rows], out["g_s"], out["s_scales"][rows], out["s_nib"][rows])
    rn = O.unpack_nibbles(out["r_codes"])
    _check_codes(r[rows], out["g_r"], out["r_scales"][rows], rn[rows])
    # d is the binary32 product (val * s) * g_s of the kept codes
    s_val = O.e4m3_value(out["s_scales"]).repeat(16, axis=1)
    dd = np.where(kept, (O.e2m1_value(out["s_nib"]) * s_val).astype(np.float32) * out["g_s"], 0)
    assert np.array_equal(d, dd.astype(np.float32))


def test_prepare_nv_zero_tensor():
    x = np.zeros((2, 64), dtype=np.uint16)
    out = O.prepare_nv(x, None, 1e-5)
    assert out["g_s"] == 1.0 and out["g_r"] == 1.0
    assert np.all(out["s_scales"] == 0) and np.all(out["r_scales"] == 0)
    assert np.all(out["s_codes"] == 0) and np.all(out["r_codes"] == 0)
    assert np.all(out["s_meta"] == 0x44)                 # ties keep the two lowest offsets


# ------------------------------------------------------------------ GEMM
def _exact_nv(codes, scales, g, K, meta=None):
    out = []
    G = Fraction(float(g))
    for row in range(codes.shape[0]):
        nibs = []
        for byte in codes[row]:
            nibs += [int(byte) & 15, int(byte) >> 4]
        if meta is not None:
            dense = [0] * K
            pos = []
            for gi in range(K // 4):
                nb = (int(meta[row, gi // 2]) >> (4 * (gi % 2))) & 15
                pos += [4 * gi + (nb & 3), 4 * gi + (nb >> 2)]
            for p, c in zip(pos, nibs):
                dense[p] = c
            nibs = dense
        row_v = []
        for k, c in enumerate(nibs):
            val = E2M1_Q[c & 7] * (-1 if c & 8 else 1)
            row_v.append(val * e4m3_exact(int(scales[row, k // 16])) * G)
        out.append(row_v)
    return out


def test_linear_nv_exact_rational():
    inp = synth.layer_inputs("decode8", seed=0, M=3, with_weight=False)
    K = 64
    x = inp["x"][:, :K]
    w = synth.linear_weight(np.random.default_rng(4), 5, K)
    act = O.prepare_nv(x, None, 1e-5)
    wc, ws, gw = O.pack_weight_nv(w)
    y, b = O.linear_nv(act, wc, ws, gw)
    S = _exact_nv(act["s_codes"], act["s_scales"], act["g_s"], K, act["s_meta"])
    R = _exact_nv(act["r_codes"], act["r_scales"], act["g_r"], K)
    W = _exact_nv(wc, ws, gw, K)
    for m in range(3):
        for n in range(5):
            ys = sum(S[m][k] * W[n][k] for k in range(K))
            yr = sum(R[m][k] * W[n][k] for k in range(K))
            bb = sum(abs(S[m][k] * W[n][k]) + abs(R[m][k] * W[n][k]) for k in range(K))
            assert abs(Fraction(y[m, n]) - (ys + yr)) <= Fraction(1, 10 ** 12) * bb
            assert abs(Fraction(b[m, n]) - bb) <= Fraction(1, 10 ** 12) * bb


def test_linear_nv_tracks_unquantised_product():
    """The residual path recovers what the backbone loses: Y is far closer to
    v deq(W)^T than the backbone alone, and within the residual's own
    quantisation error."""
    inp = synth.layer_inputs("decode8", seed=2, M=4, with_weight=False)
    w = synth.linear_weight(np.random.default_rng(9), 64, inp["K"])
    act = O.prepare_nv(inp["x"], None, 1e-5)
    wc, ws, gw = O.pack_weight_nv(w)
    y, _ = O.linear_nv(act, wc, ws, gw)
    dw = O.dequant_nv(ws, O.unpack_nibbles(wc), gw)
    exact = act["v"].astype(np.float64) @ dw.T
    rq = O.dequant_nv(act["r_scales"], O.unpack_nibbles(act["r_codes"]), act["g_r"])
    bound = np.abs(rq - act["r"].astype(np.float64)) @ np.abs(dw).T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9) + 1e-12)
    back = dict(act, r_codes=np.zeros_like(act["r_codes"]))
    ys, _ = O.linear_nv(back, wc, ws, gw)
    assert np.linalg.norm(y - exact) < 0.5 * np.linalg.norm(ys - exact)
