"""GPU parity of the fused preparation and the weight pack: every byte of
masks, codes and scales equals the CPU oracle's, on every workload shape and
on the edge cases of the method."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_prep_equal, dev_bf16, untile_act, untile_weight

pytestmark = pytest.mark.gpu


def run_prep(x_bits, gamma_bits, eps=1e-5, ldx=None):
    import torch
    M, K = x_bits.shape
    if ldx is not None and ldx != K:
        pad = np.zeros((M, ldx), dtype=np.uint16)
        pad[:, :K] = x_bits
        xd = dev_bf16(pad)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    g = dev_bf16(gamma_bits) if gamma_bits is not None else None
    act = sq.sharq_prepare(xd, g, eps)
    torch.cuda.synchronize()
    return untile_act(act.host(), M, K)


CASES = [("tiny", 0), ("qkv", 0), ("qkv", 1), ("qkv", 2), ("down", 0),
         ("decode1", 0), ("decode8", 0), ("decode32", 0), ("decode64", 0)]


@pytest.mark.parametrize("name,seed", CASES)
def test_prep_workloads(name, seed):
    print(f"prep {name} seed {seed}", flush=True)
    inp = synth.layer_inputs(name, seed=seed, with_weight=False)
    ref = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    got = run_prep(inp["x"], inp["gamma"], inp["eps"])
    assert_prep_equal(got, ref, f"{name}/{seed}")


def test_prep_moe_rows():
    print("prep moe", flush=True)
    moe = synth.moe_inputs(seed=0, with_weights=False)
    for key in ("x_tok", "x_down"):
        ref = O.prepare(moe[key], None)
        got = run_prep(moe[key], None)
        assert_prep_equal(got, ref, key)


def _edge_rows(K, rng):
    rows = []
    rows.append(np.zeros(K, np.float32))                              # all zero
    z = np.zeros(K, np.float32); z[1::2] = -0.0; rows.append(z)       # signed zeros
    rows.append(np.full(K, 1.5, np.float32))                          # all ties
    rows.append(np.tile(np.array([2, -2, 2, -2], np.float32), K // 4))  # ties with signs
    rows.append(rng.standard_normal(K).astype(np.float32) * np.float32(1e-39))   # subnormal bf16
    t = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -120); rows.append(t)   # tiny normals
    u = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** -68); rows.append(u)    # squares below 2^-126
    big = rng.standard_normal(K).astype(np.float32) * np.float32(1e37); rows.append(big)      # huge
    o = rng.standard_normal(K).astype(np.float32); o[::32] = 3e4; rows.append(o)               # outliers
    s = rng.standard_normal(K).astype(np.float32); s[5] = 7.0 * 2 ** 10; rows.append(s)
    q = (rng.integers(-12, 13, K) * 0.5).astype(np.float32); rows.append(q)                     # grid values
    return synth.bf16_bits_from_f32(np.stack(rows))


@pytest.mark.parametrize("K", [32, 96, 256, 544, 4096, 8192])
@pytest.mark.parametrize("norm", [False, True])
def test_prep_edge_rows(K, norm):
    print(f"prep edge K={K} norm={norm}", flush=True)
    rng = np.random.default_rng(K)
    x = _edge_rows(K, rng)
    g = synth.norm_weight(rng, K) if norm else None
    ref = O.prepare(x, g, 1e-5)
    got = run_prep(x, g, 1e-5)
    assert_prep_equal(got, ref, f"edge K={K} norm={norm}")


@pytest.mark.parametrize("M,K,ldx,norm", [(1, 4096, 4096, True), (3, 32768, 32768, True),
                                          (5, 16384, 16384, True), (7, 2048, 2056, True),
                                          (9, 768, 800, False), (130, 14336, 14336, False),
                                          # K slices without RMSNorm with a ragged last slice and K tail
                                          (40, 4128, 4136, False), (17, 6176, 6176, False)])
def test_prep_shapes(M, K, ldx, norm):
    print(f"prep shape M={M} K={K} ldx={ldx} norm={norm}", flush=True)
    rng = np.random.default_rng(M * K)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    ref = O.prepare(x, g, 1e-5)
    got = run_prep(x, g, 1e-5, ldx=ldx)
    assert_prep_equal(got, ref, f"M={M} K={K}")


@pytest.mark.parametrize("M,K,ldx", [(13, 4096, 4096), (21, 4160, 4168), (11, 6176, 6176), (3, 8192, 8200),
                                     (29, 1056, 1056)])
def test_prep_norm_signed_gamma(M, K, ldx):
    """RMSNorm rows with gamma of both signs (a negative gamma must not turn the
    padding rows' zero input into -0), a zero row among them, ragged M and K
    tiles, one and two blocks per lane."""
    print(f"prep signed gamma M={M} K={K}", flush=True)
    rng = np.random.default_rng(M * 7 + K)
    x = synth.outlier_activations(rng, M, K)
    x[M // 2] = 0
    g = synth.bf16_bits_from_f32((rng.uniform(0.5, 1.5, K) * rng.choice([-1.0, 1.0], K)).astype(np.float32))
    ref = O.prepare(x, g, 1e-5)
    got = run_prep(x, g, 1e-5, ldx=ldx)
    assert_prep_equal(got, ref, f"signed gamma M={M} K={K}")


def test_prep_eps_values():
    inp = synth.layer_inputs("tiny", seed=0, with_weight=False)
    for eps in (1e-6, 0.5, 0.0):
        ref = O.prepare(inp["x"], inp["gamma"], eps)
        got = run_prep(inp["x"], inp["gamma"], eps)
        assert_prep_equal(got, ref, f"eps={eps}")


def test_prep_deterministic():
    inp = synth.layer_inputs("qkv", seed=0, with_weight=False)
    a = run_prep(inp["x"], inp["gamma"])
    b = run_prep(inp["x"], inp["gamma"])
    for f in a:
        assert np.array_equal(a[f], b[f])


def test_prep_empty():
    import torch
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    act = sq.sharq_prepare(x, None)
    assert act.M == 0 and act.s_codes.numel() == 0


@pytest.mark.parametrize("name", ["tiny", "qkv", "down"])
def test_pack_weight(name):
    import torch
    print(f"pack {name}", flush=True)
    inp = synth.layer_inputs(name, seed=0)
    wc, ws = O.pack_weight(inp["w"])
    w = sq.sharq_pack_weight(dev_bf16(inp["w"]))
    torch.cuda.synchronize()
    gc, gs = untile_weight(w.codes.cpu().numpy(), w.scales.cpu().numpy(), inp["N"], inp["K"])
    assert np.array_equal(gc, wc)
    assert np.array_equal(gs, ws)
    assert w.desc.view[0].base == w.desc.view[1].base == w.scales.data_ptr()


def test_pack_weight_edges():
    import torch
    rng = np.random.default_rng(3)
    w = _edge_rows(96, rng)
    wc, ws = O.pack_weight(w)
    p = sq.sharq_pack_weight(dev_bf16(w))
    torch.cuda.synchronize()
    gc, gs = untile_weight(p.codes.cpu().numpy(), p.scales.cpu().numpy(), w.shape[0], w.shape[1])
    assert np.array_equal(gc, wc)
    assert np.array_equal(gs, ws)
