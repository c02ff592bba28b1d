"""Pins for the oracle's plain FP4 linear (the dense FP4 baseline: no backbone,
MXFP4 of the normalised row, one GEMM).  Expected values come from exact
rationals and the MX definition (E = floor(log2 amax) - 2, E2M1 nearest with
ties to the even code), written independently of the oracle's vectorised code."""
from fractions import Fraction

import numpy as np

from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O

E2M1_Q = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
          Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _floor_log2(q: Fraction) -> int:
    e = 0
    while q >= 2:
        q /= 2
        e += 1
    while q < 1:
        q *= 2
        e -= 1
    return e


def _code(t: Fraction, negative: bool) -> int:
    d = [abs(abs(t) - g) for g in E2M1_Q]
    best = min(d)
    c = [i for i, x in enumerate(d) if x == best]
    code = c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]
    return code | (8 if negative else 0)


def test_prepare_dense_exact_rationals():
    inp = synth.layer_inputs("tiny", seed=0)
    x, g = inp["x"][:3], inp["gamma"]
    out = O.prepare_dense(x, g, inp["eps"])
    v = out["v"]
    nib = O.unpack_nibbles(out["r_codes"])
    for r in range(3):
        for b in range(v.shape[1] // 32):
            blk = [Fraction(float(t)) for t in v[r, 32 * b:32 * b + 32]]
            amax = max(abs(t) for t in blk)
            e = _floor_log2(amax) - 2 if amax else -127
            assert int(out["r_scales"][r, b]) == e + 127
            for i, t in enumerate(blk):
                want = _code(t / Fraction(2) ** e, bool(np.signbit(v[r, 32 * b + i])))
                assert nib[r, 32 * b + i] == want, (r, b, i)


def test_dense_reproduces_grid_inputs():
    """Rows already on the MXFP4 grid (E2M1 values times 2^e, a 6 * 2^e in every
    block): the codes are the inputs' own codes and deq(Q(v)) == v exactly."""
    rng = np.random.default_rng(2)
    M, K = 4, 128
    nib = (rng.integers(0, 8, (M, K)) | (rng.integers(0, 2, (M, K)) << 3)).astype(np.uint8)
    nib[:, ::32] = 7                                    # block maximum 6 * 2^e
    e = rng.integers(-12, 12, (M, K // 32))
    vals = (O.e2m1_value(nib).reshape(M, K // 32, 32) * np.exp2(e)[..., None]).reshape(M, K)
    x = synth.bf16_bits_from_f32(vals.astype(np.float32))
    out = O.prepare_dense(x, None, 1e-5)
    got = O.unpack_nibbles(out["r_codes"])
    # a negative zero input keeps its sign code; compare values, then codes of nonzeros
    assert np.array_equal(O.deq_dense(out["r_codes"], out["r_scales"]), vals)
    nz = vals != 0
    assert np.array_equal(got[nz], nib[nz])
    assert np.array_equal(out["r_scales"].astype(np.int64), e + 127)


def test_linear_dense_exact_and_bound():
    inp = synth.layer_inputs("qkv", seed=1, M=3, with_weight=False)
    K = 64
    x = inp["x"][:, :K]
    w = synth.linear_weight(np.random.default_rng(7), 5, K)
    act = O.prepare_dense(x, None, 1e-5)
    wc, ws = O.pack_weight(w)
    y, b = O.linear_dense(act, wc, ws)

    def rows(codes, scales):
        out = []
        for r in range(codes.shape[0]):
            nibs = []
            for byte in codes[r]:
                nibs += [int(byte) & 15, int(byte) >> 4]
            out.append([E2M1_Q[c & 7] * (-1 if c & 8 else 1) * Fraction(2) ** (int(scales[r, k // 32]) - 127)
                        for k, c in enumerate(nibs)])
        return out
    A, W = rows(act["r_codes"], act["r_scales"]), rows(wc, ws)
    for m in range(3):
        for n in range(5):
            ex = sum(A[m][k] * W[n][k] for k in range(K))
            bb = sum(abs(A[m][k] * W[n][k]) for k in range(K))
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(1, 10 ** 12) * bb
            assert abs(Fraction(b[m, n]) - bb) <= Fraction(1, 10 ** 12) * bb
    # quantisation error bound: |Y - v W^T| <= sum |Q(v) - v| |W|
    dw = O.deq_dense(wc, ws)
    dv = O.deq_dense(act["r_codes"], act["r_scales"])
    exact = act["v"].astype(np.float64) @ dw.T
    bound = np.abs(dv - act["v"]) @ np.abs(dw).T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-12) + 1e-12)
