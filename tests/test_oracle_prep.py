"""Pins for the oracle's preparation steps: RMSNorm, 2:4 mask, S/R quantisation,
residual.  Expected values come from hand derivation (tests/golden), closed
forms, exhaustive brute force and invariants that the method fixes."""
import itertools
import json
import os

import numpy as np
import pytest

from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _vals(lst):
    return np.array([-0.0 if v == "-0" else float(v) for v in lst], dtype=np.float32)


# ---------------------------------------------------------------- RMSNorm
def test_pairwise_tree_order():
    t = np.float32(2.0 ** 24)
    # (2^24 + 1) rounds to 2^24 (tie to even), (1 + 1) = 2, then 2^24 + 2 is exact.
    # A left-to-right sum would give 2^24: this pins the pairwise order.
    assert O.pairwise_tree_sum_f32(np.array([t, 1, 1, 1], dtype=np.float32)) == t + 2
    # K = 6 pads to 8: ((a+b)+(c+d)) + ((e+f)+(0+0))
    q = np.array([t, 1, 1, 1, 1, 1], dtype=np.float32)
    assert O.pairwise_tree_sum_f32(q) == t + 4
    # integer-valued rows: every order gives the exact sum
    rng = np.random.default_rng(0)
    q = rng.integers(0, 1000, (50, 777)).astype(np.float32)
    assert np.array_equal(O.pairwise_tree_sum_f32(q), q.sum(-1, dtype=np.float64).astype(np.float32))


def test_rmsnorm_constant_row_closed_form():
    K = 4096
    for c in (1.0, 2.0, 0.5, 3.0, 40.0):
        x = synth.bf16_bits_from_f32(np.full((1, K), c, dtype=np.float32))
        g = synth.bf16_bits_from_f32(np.ones(K, dtype=np.float32))
        v = O.rmsnorm(x, g, 1e-5)
        ref = c / np.sqrt(c * c + np.float64(np.float32(1e-5)))
        ulp = np.spacing(np.float32(ref))
        assert np.all(np.abs(v.astype(np.float64) - ref) <= 2 * ulp)


def test_rmsnorm_against_fp64_formula():
    inp = synth.layer_inputs("qkv", seed=0, M=8, with_weight=False)
    v = O.rmsnorm(inp["x"], inp["gamma"], inp["eps"])
    x = O.widen_bf16(inp["x"]).astype(np.float64)
    g = O.widen_bf16(inp["gamma"]).astype(np.float64)
    ref = x / np.sqrt((x * x).mean(-1, keepdims=True) + np.float64(np.float32(1e-5))) * g
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(v - ref) <= 4 * ulp)


def test_rmsnorm_identity_without_gamma():
    x = synth.layer_inputs("down", seed=0, M=3, with_weight=False)["x"]
    assert np.array_equal(O.rmsnorm(x, None, 1e-5).view(np.uint32),
                          O.widen_bf16(x).view(np.uint32))


# ---------------------------------------------------------------- mask
def _brute_keep(vals, n):
    """The kept set is the unique n-subset whose every member beats every
    non-member (|a| larger, or equal magnitude and lower index)."""
    m = len(vals)
    mags = [abs(float(v)) for v in vals]

    def beats(i, k):
        return mags[i] > mags[k] or (mags[i] == mags[k] and i < k)

    found = [set(c) for c in itertools.combinations(range(m), n)
             if all(beats(i, k) for i in c for k in range(m) if k not in c)]
    assert len(found) == 1
    return found[0]


def test_mask_bruteforce_all_tuples():
    alphabet = [0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0]
    tuples = np.array(list(itertools.product(alphabet, repeat=4)), dtype=np.float32)
    kept = O.nm_mask(tuples, 2, 4)
    for row, k in zip(tuples, kept):
        assert set(np.nonzero(k)[0]) == _brute_keep(row, 2)


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (2, 8), (4, 8)])
def test_mask_general_nm_invariants(n, m):
    rng = np.random.default_rng(n * 10 + m)
    v = rng.integers(-3, 4, (64, 16 * m)).astype(np.float32)
    kept = O.nm_mask(v, n, m)
    g = kept.reshape(64, -1, m)
    assert np.all(g.sum(-1) == n)
    a = np.abs(v).reshape(64, -1, m)
    kmin = np.where(g, a, np.inf).min(-1)
    dmax = np.where(~g, a, -np.inf).max(-1)
    assert np.all(kmin >= dmax)


# ---------------------------------------------------------------- golden row
def test_hand_worked_row():
    G = json.load(open(os.path.join(GOLDEN, "hand_row_k32.json")))
    x = synth.bf16_bits_from_f32(_vals(G["x"]))[None]
    assert np.array_equal(O.widen_bf16(x)[0].view(np.uint32), _vals(G["x"]).view(np.uint32))
    out = O.prepare(x, None, 1e-5)
    kept = np.zeros(32, dtype=bool)
    for gi, (a, b) in enumerate(G["kept_offsets"]):
        kept[4 * gi + a] = kept[4 * gi + b] = True
    assert np.array_equal(out["kept"][0], kept)
    assert list(out["s_meta"][0]) == G["s_meta"]
    assert list(out["s_scales"][0]) == G["s_scales"]
    assert list(out["s_codes"][0]) == G["s_codes"]
    assert np.array_equal(out["d"][0].view(np.uint32), _vals(G["d"]).view(np.uint32))
    assert np.array_equal(out["r"][0].view(np.uint32), _vals(G["r"]).view(np.uint32))
    assert list(out["r_scales"][0]) == G["r_scales"]
    assert list(out["r_codes"][0]) == G["r_codes"]


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("name,M", [("tiny", 16), ("qkv", 24), ("down", 6), ("decode1", 1)])
def test_prepare_invariants(name, M):
    inp = synth.layer_inputs(name, seed=1, M=M, with_weight=False)
    out = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    v, d, r, kept = out["v"], out["d"], out["r"], out["kept"]
    K = v.shape[1]
    # exactly two kept per group; kept magnitudes dominate dropped ones
    g = kept.reshape(M, K // 4, 4)
    assert np.all(g.sum(-1) == 2)
    a = np.abs(v).reshape(M, K // 4, 4)
    assert np.all(np.where(g, a, np.inf).min(-1) >= np.where(~g, a, -np.inf).max(-1))
    # residual is exact: d + r == v bit for bit (signed zeros compare by value)
    assert np.array_equal(d + r, v)
    assert np.array_equal((d.astype(np.float64) + r.astype(np.float64)), v.astype(np.float64))
    # r is zero-or-v: non-kept positions carry v itself
    assert np.array_equal(r[~kept].view(np.uint32), v[~kept].view(np.uint32))
    # the S scale equals the scale of the unmasked block (block max is always kept)
    sv, _ = O.quantize_mx(v)
    assert np.array_equal(out["s_scales"], sv)
    # metadata decodes back to the mask
    assert np.array_equal(O.unpack_meta_24(out["s_meta"], K), kept)
    # sizes
    assert out["s_codes"].shape == (M, K // 4) and out["r_codes"].shape == (M, K // 2)
    assert out["s_scales"].shape == (M, K // 32) == out["r_scales"].shape


def test_residual_vanishes_on_grid_inputs():
    """X with two nonzeros per group, already on the MXFP4 grid with a block max
    of 6 * 2^e: the backbone is exact, R == 0, S codes are X's codes."""
    rng = np.random.default_rng(5)
    M, K = 4, 128
    keep = np.zeros((M, K // 4, 4), dtype=bool)
    for i in range(M):
        for j in range(K // 4):
            keep[i, j, rng.choice(4, 2, replace=False)] = True
    keep = keep.reshape(M, K)
    mag = rng.integers(1, 8, (M, K)).astype(np.uint8)          # nonzero magnitudes
    sign = rng.integers(0, 2, (M, K)).astype(np.uint8) << 3
    nib = np.where(keep, mag | sign, 0).astype(np.uint8)
    for b in range(K // 32):                                     # a 6 in every block
        first = keep[:, 32 * b:32 * b + 32].argmax(-1)
        nib[np.arange(M), 32 * b + first] = 7
    e = rng.integers(-10, 10, (M, K // 32))
    vals = O.e2m1_value(nib).reshape(M, K // 32, 32) * np.exp2(e)[..., None]
    x = synth.bf16_bits_from_f32(vals.reshape(M, K).astype(np.float32))
    out = O.prepare(x, None, 1e-5)
    assert np.array_equal(out["kept"], keep)
    assert np.array_equal(out["s_nib"][keep], nib[keep])
    assert np.all(out["r"] == 0)
    assert np.all(out["r_scales"] == 0)
    assert np.array_equal(out["s_scales"].astype(np.int64), e + 127)
