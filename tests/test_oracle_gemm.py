"""Pins for the oracle's dual GEMM: hand-derived values, exact rational
arithmetic on tiny shapes, the path split and the R == 0 special case."""
import json
import os
from fractions import Fraction

import numpy as np

from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_Q = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
          Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _dec(nib):
    v = E2M1_Q[nib & 7]
    return -v if nib & 8 else v


def _exact_rows(codes, scales, K, meta=None):
    """Decode bytes to exact rationals, written independently of the oracle."""
    out = []
    for row in range(codes.shape[0]):
        nibs = []
        for byte in codes[row]:
            nibs += [int(byte) & 15, int(byte) >> 4]
        if meta is not None:                       # 2:4 compressed: scatter by offsets
            dense = [0] * K
            pos = []
            for gi in range(K // 4):
                nb = (int(meta[row, gi // 2]) >> (4 * (gi % 2))) & 15
                pos += [4 * gi + (nb & 3), 4 * gi + (nb >> 2)]
            for p, c in zip(pos, nibs):
                dense[p] = c
            nibs = dense
        vals = [_dec(c) * Fraction(2) ** (int(scales[row, k // 32]) - 127) for k, c in enumerate(nibs)]
        out.append(vals)
    return out


def test_hand_worked_gemm():
    G = json.load(open(os.path.join(GOLDEN, "hand_row_k32.json")))
    x = synth.bf16_bits_from_f32(np.array(
        [-0.0 if v == "-0" else float(v) for v in G["x"]], dtype=np.float32))[None]
    act = O.prepare(x, None, 1e-5)
    w = synth.bf16_bits_from_f32(np.ones((1, 32), dtype=np.float32))
    wc, ws = O.pack_weight(w)
    gw = G["gemm_w_row_all_ones"]
    assert ws[0, 0] == gw["w_scale"] and np.all(O.unpack_nibbles(wc) == gw["w_code"])
    y, b = O.linear(act, wc, ws)
    assert y[0, 0] == gw["y"] and b[0, 0] == gw["bound"]
    ds = O.deq_sparse(act["s_codes"], act["s_meta"], act["s_scales"], 32)
    dr = O.deq_dense(act["r_codes"], act["r_scales"])
    assert ds.sum() == gw["y_sparse"] and dr.sum() == gw["y_dense"]


def test_tiny_gemm_exact_rational():
    inp = synth.layer_inputs("tiny", seed=0, M=3)
    K = inp["K"]
    w = inp["w"][:5]
    act = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(w)
    y, b = O.linear(act, wc, ws)
    S = _exact_rows(act["s_codes"], act["s_scales"], K, meta=act["s_meta"])
    R = _exact_rows(act["r_codes"], act["r_scales"], K)
    W = _exact_rows(wc, ws, K)
    for m in range(3):
        for n in range(5):
            ex = sum(s * w_ for s, w_ in zip(S[m], W[n])) + sum(r * w_ for r, w_ in zip(R[m], W[n]))
            bd = sum(abs(s * w_) for s, w_ in zip(S[m], W[n])) + sum(abs(r * w_) for r, w_ in zip(R[m], W[n]))
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(1, 10 ** 12) * bd
            assert abs(Fraction(b[m, n]) - bd) <= Fraction(1, 10 ** 12) * bd
    # the exact backbone + exact residual reproduce the normalised input
    # (D^S + R == v), so the dense path's error is only R's quantisation error
    v = act["v"].astype(np.float64)
    for m in range(3):
        for k in range(0, K, 17):
            assert Fraction(float(act["d"][m, k])) + Fraction(float(act["r"][m, k])) == Fraction(float(v[m, k]))
            assert Fraction(float(act["d"][m, k])) == S[m][k]


def test_gemm_approximates_unquantised_product():
    """The dense residual path compensates mask loss and backbone quantisation
    error: |Y - v deq(W)^T| <= sum_k |deq(Q(R)) - R| |D^W|."""
    inp = synth.layer_inputs("qkv", seed=2, M=4, with_weight=False)
    rng = np.random.default_rng(9)
    w = synth.linear_weight(rng, 64, inp["K"])
    act = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(w)
    y, _ = O.linear(act, wc, ws)
    dw = O.deq_dense(wc, ws)
    exact = act["v"].astype(np.float64) @ dw.T
    rq = O.deq_dense(act["r_codes"], act["r_scales"])
    bound = np.abs(rq - act["r"].astype(np.float64)) @ np.abs(dw).T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-12) + 1e-12)
    # and it is much closer than the backbone alone
    ys = O.deq_sparse(act["s_codes"], act["s_meta"], act["s_scales"], inp["K"]) @ dw.T
    assert np.linalg.norm(y - exact) < 0.5 * np.linalg.norm(ys - exact)


def test_within_tolerance_rule():
    ref = np.array([1.0, -2.0, 0.0])
    bound = np.array([10.0, 10.0, 0.0])
    ok = O.within_tolerance(np.array([1.0 + 9e-5, -2.0 - 1.1e-4, 9e-7]), ref, bound)
    assert list(ok) == [True, False, True]
