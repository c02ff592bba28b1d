"""Pins for the oracle's fusion-ablation pieces: bf16 rounding (exact rationals,
ties to even), the unfused RMSNorm, and the two GEMM paths on their own."""
from fractions import Fraction

import numpy as np

from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O


def _bf16_value(bits) -> Fraction:
    return Fraction(float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]))


def test_round_bf16_against_exact_rationals():
    rng = np.random.default_rng(4)
    base = rng.integers(0, 0x7F7F, 300).astype(np.uint32) << 16      # finite positive bf16
    vals = []
    for b in base:
        for d in (0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x10000 - 0x8000):
            vals.append(int(b) + d)
    f = np.array(vals, dtype=np.uint32).view(np.float32)
    f = np.concatenate([f, -f])
    got = O.round_bf16(f)
    for x, g in zip(f, got):
        q = Fraction(float(x))
        lo = np.array([np.float32(x)], dtype=np.float32).view(np.uint32)[0] >> 16
        sign = 0x8000 if q < 0 else 0
        cands = [int(lo), int(lo) + 1]
        dist = [abs(_bf16_value(c) - q) for c in cands]
        if dist[0] != dist[1]:
            want = cands[int(dist[1] < dist[0])]
        else:
            want = [c for c in cands if c % 2 == 0][0]
        assert int(g) == want, (float(x), hex(int(g)), hex(want), sign)


def test_round_bf16_roundtrip_and_closed_forms():
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(O.round_bf16(f), b)
    # ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert O.round_bf16(np.float32(1 + 2 ** -8)) == 0x3F80
    assert O.round_bf16(np.float32(1 + 3 * 2 ** -8)) == 0x3F82   # halfway, upper is even


def test_unfused_rmsnorm_is_the_rounded_fused_row():
    inp = synth.layer_inputs("qkv", seed=3, M=4, with_weight=False)
    got = O.rmsnorm_bf16(inp["x"], inp["gamma"], inp["eps"])
    v = O.rmsnorm(inp["x"], inp["gamma"], inp["eps"])
    back = (got.astype(np.uint32) << 16).view(np.float32)
    # within half a bf16 ulp of v, and exactly v where v is already a bf16 value
    ulp = np.exp2(np.floor(np.log2(np.abs(v.astype(np.float64)) + 1e-300)) - 7)
    assert np.all(np.abs(back.astype(np.float64) - v) <= ulp / 2)
    exact = (v.view(np.uint32) & 0xFFFF) == 0
    assert np.array_equal(back[exact], v[exact])


def test_paths_sum_to_the_fused_gemm():
    inp = synth.layer_inputs("tiny", seed=0)
    act = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(inp["w"])
    ys, yr, b = O.linear_paths(act, wc, ws)
    y, b2 = O.linear(act, wc, ws)
    assert np.allclose(ys + yr, y, rtol=0, atol=1e-12 * b.max())
    assert np.array_equal(b, b2)
    # the backbone path alone is the plain FP4 GEMM of the dense backbone codes
    dense_s = dict(r_codes=O.pack_nibbles(act["s_nib"]), r_scales=act["s_scales"])
    ys2, _ = O.linear_dense(dense_s, wc, ws)
    assert np.allclose(ys2, ys, rtol=0, atol=1e-12 * b.max())


def test_gate_up_interleave_and_split():
    rng = np.random.default_rng(6)
    g = rng.standard_normal((32, 8))
    u = rng.standard_normal((32, 8))
    w = O.interleave_gate_up(g, u)
    assert w.shape == (64, 8)
    assert np.array_equal(w[0:16], g[0:16]) and np.array_equal(w[16:32], u[0:16])
    assert np.array_equal(w[32:48], g[16:32]) and np.array_equal(w[48:64], u[16:32])
    # a layer output's columns follow the weight rows: splitting inverts the interleave
    y = w.T                                       # [8, 64]: column n is weight row n
    gg, uu = O.split_gate_up(y)
    assert np.array_equal(gg, g.T) and np.array_equal(uu, u.T)


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
    assert O.silu(-800.0) == 0.0 and O.silu(800.0) == 800.0          # saturation both ways
    x = np.linspace(-6, 6, 101)
    assert np.allclose(O.silu(x) - O.silu(-x), x)                      # silu(x) - silu(-x) = x


def test_swiglu_equals_split_layers():
    inp = synth.layer_inputs("tiny", seed=1)
    rng = np.random.default_rng(3)
    wg = synth.linear_weight(rng, 32, inp["K"])
    wu = synth.linear_weight(rng, 32, inp["K"])
    act = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(O.interleave_gate_up(wg, wu))
    h, bg, bu, g, u = O.linear_swiglu(act, wc, ws)
    gc, gs = O.pack_weight(wg)
    uc, us = O.pack_weight(wu)
    g2, _ = O.linear(act, gc, gs)
    u2, _ = O.linear(act, uc, us)
    assert np.allclose(g, g2, rtol=0, atol=1e-12) and np.allclose(u, u2, rtol=0, atol=1e-12)
    assert np.allclose(h, O.silu(g2) * u2, rtol=1e-12, atol=1e-15)


def test_swiglu_bound_covers_bf16_rounding():
    """The bound must admit the worst bf16 rounding: a value just above a power of
    two rounds by up to 2^-8 relative (half an ulp of 8 significant bits)."""
    h = np.float32(1 + 2 ** -8)                       # halfway between bf16 1 and 1 + 2^-7
    got = (np.array([O.round_bf16(h)], dtype=np.uint32) << 16).view(np.float32)[0]
    err = abs(float(got) - float(h))
    assert err == 2 ** -8
    g = np.array([30.0])                              # SiLU(30) = 30 to 1e-12
    u = np.array([float(h) / 30.0])
    b = O.swiglu_bound(g, u, np.zeros(1), np.zeros(1), rel=0.0, abs_=0.0)
    assert b[0] >= err * (1 - 1e-9)


def test_residual_add_closed_forms():
    x = np.array([0x3F80, 0xBF80, 0x4000, 0x0000], dtype=np.uint16)      # 1, -1, 2, 0
    y = np.array([0.5, 1.0, 2 ** -8, -0.0], dtype=np.float32)
    got = O.residual_add_bf16(x, y)
    # 1.5 exact; -1 + 1 = +0; 2 + 2^-8 rounds to 2 (below half an ulp, 2^-7); 0 + -0 = +0
    assert list(got) == [0x3FC0, 0x0000, 0x4000, 0x0000]
