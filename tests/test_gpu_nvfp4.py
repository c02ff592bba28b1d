"""GPU parity of the NVFP4-style path (E4M3 scale per 16, binary32 tensor
scales): preparation and weight packing byte-exact against the oracle (codes,
metadata, block scales, tensor scales), the dual GEMM within
1e-5 * sum|terms| + 1e-6 of the float64 oracle."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import (assert_linear_close, assert_prep_equal, dev_bf16, untile_act_nv,
                               untile_weight_nv)

pytestmark = pytest.mark.gpu
NV = sq.FMT_NVFP4


def run_prep(x, gamma, eps=1e-5, ldx=None):
    import torch
    M, K = x.shape
    if ldx is not None and ldx != K:
        buf = np.zeros((M, ldx), dtype=np.uint16)
        buf[:, :K] = x
        xd = dev_bf16(buf)[:, :K]
    else:
        xd = dev_bf16(x)
    act = sq.sharq_prepare(xd, dev_bf16(gamma) if gamma is not None else None, eps, fmt=NV)
    torch.cuda.synchronize()
    return act


def check_prep(act, ref, M, K, label):
    got = untile_act_nv(act.host(), M, K)
    assert_prep_equal(got, ref, label)
    assert got["g_s"] == ref["g_s"] and got["g_r"] == ref["g_r"], (label, got["g_s"], ref["g_s"], got["g_r"], ref["g_r"])


@pytest.mark.parametrize("M,K,ldx,norm", [(1, 4096, 4096, False), (8, 4096, 4096, False), (37, 96, 104, True),
                                          (64, 4096, 4096, False), (130, 768, 768, True), (3, 1376, 1376, False),
                                          (5, 32768, 32768, True),
                                          # one workgroup for all three phases (at most 512 chunks of 32)
                                          (4, 4096, 4104, True), (16, 1024, 1024, True), (13, 1056, 1056, False),
                                          # two launches: phase 2 scans X for max |x| (no RMSNorm, small X)
                                          (9, 2080, 2088, False)])
def test_nv_prep_shapes(M, K, ldx, norm):
    print(f"nv prep M={M} K={K} ldx={ldx} norm={norm}", flush=True)
    rng = np.random.default_rng(M * K + 7)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    ref = O.prepare_nv(x, g, 1e-5)
    act = run_prep(x, g, ldx=ldx)
    check_prep(act, ref, M, K, f"M={M} K={K}")


def test_nv_prep_zero_and_tiny_rows():
    """An all-zero tensor (tensor scales 1, every code and scale zero) and a
    tensor whose rows span many binades (small blocks get subnormal or zero
    E4M3 scales)."""
    print("nv prep zero", flush=True)
    x = np.zeros((4, 256), dtype=np.uint16)
    check_prep(run_prep(x, None), O.prepare_nv(x, None), 4, 256, "zero")
    rng = np.random.default_rng(3)
    v = rng.standard_normal((20, 512)) * np.exp2(rng.uniform(-30, 4, (20, 32))).repeat(16, axis=1)
    x = synth.bf16_bits_from_f32(v.astype(np.float32))
    check_prep(run_prep(x, None), O.prepare_nv(x, None), 20, 512, "binades")


@pytest.mark.parametrize("N,K", [(53, 96), (4096, 4096), (200, 1376)])
def test_nv_pack_weight(N, K):
    import torch
    print(f"nv pack N={N} K={K}", flush=True)
    w = synth.linear_weight(np.random.default_rng(N + K), N, K)
    wt = sq.sharq_pack_weight(dev_bf16(w), fmt=NV)
    torch.cuda.synchronize()
    codes, scales, g = untile_weight_nv(wt.codes.cpu().numpy(), wt.scales.cpu().numpy(), N, K)
    rc, rs, rg = O.pack_weight_nv(w)
    assert g == rg
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def tie_tensor(rng, rows, K, k=-12):
    """bf16 bits of a tensor whose every 16-block quotient u / (s g) is an E2M1
    decision point (0.25, 0.75, ... 5: exact ties) or grid value: the tensor
    maximum 2688 * 2^k makes g = 2^k, each block's maximum 6 * s0 * 2^k makes
    its E4M3 scale s0, and its other elements are m * s0 * 2^k with random
    signs (at most 7 significant bits: exact in bf16)."""
    e4m3 = [0.5, 0.625, 0.75, 1.0, 1.125, 1.5, 2.0, 3.5, 7.0, 12.0, 40.0, 448.0]
    ms = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 4.0]
    v = np.zeros((rows, K))
    for r in range(rows):
        for b in range(K // 16):
            s0 = 448.0 if (r, b) == (0, 0) else e4m3[rng.integers(len(e4m3) - 1)]
            t = s0 * 2.0 ** k
            blk = rng.choice(ms, 16) * t * rng.choice([-1.0, 1.0], 16)
            blk[rng.integers(16)] = 6.0 * t * rng.choice([-1.0, 1.0])
            v[r, 16 * b:16 * b + 16] = blk
    v[0, 0] = 2688.0 * 2.0 ** k
    return synth.bf16_bits_from_f32(v.astype(np.float32))


def test_nv_exact_quotient_ties():
    """Block quotients exactly on the E2M1 decision points (ties to the even
    code) for the backbone and the weight, every block; the residual's
    quotients follow from them."""
    import torch
    print("nv ties", flush=True)
    rng = np.random.default_rng(11)
    x = tie_tensor(rng, 16, 512)
    ref = O.prepare_nv(x, None)
    assert ref["g_s"] == np.float32(2.0 ** -12)
    check_prep(run_prep(x, None), ref, 16, 512, "ties")
    w = tie_tensor(rng, 48, 256)
    wt = sq.sharq_pack_weight(dev_bf16(w), fmt=NV)
    torch.cuda.synchronize()
    codes, scales, g = untile_weight_nv(wt.codes.cpu().numpy(), wt.scales.cpu().numpy(), 48, 256)
    rc, rs, rg = O.pack_weight_nv(w)
    assert g == rg == np.float32(2.0 ** -12)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def nv_layer(x, gamma, w, out_dtype=sq.OUT_F32):
    import torch
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(gamma) if gamma is not None else None, 1e-5, fmt=NV)
    wt = sq.sharq_pack_weight(dev_bf16(w), fmt=NV)
    y = sq.sharq_linear(act, wt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return act, wt, y


@pytest.mark.parametrize("M,K,N,norm", [(1, 4096, 4096, False), (37, 96, 53, True), (130, 768, 200, False),
                                        (5, 1376, 100, False), (17, 2048, 272, True), (64, 256, 48, False),
                                        # two and four weight column blocks per workgroup, the last group
                                        # partly past N
                                        (63, 1056, 2025, False), (64, 512, 4100, True), (32, 1024, 4096, False),
                                        # two column blocks on 16 waves with a partial row block
                                        (20, 512, 4096, True)])
def test_nv_linear_full(M, K, N, norm):
    print(f"nv linear M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M + K + N + 1)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    act, wt, y = nv_layer(x, g, w)
    ref = O.prepare_nv(x, g, 1e-5)
    check_prep(act, ref, M, K, f"M={M}")
    wc, ws, gw = O.pack_weight_nv(w)
    yr, b = O.linear_nv(ref, wc, ws, gw)
    assert_linear_close(y.cpu().numpy(), yr, b, f"nv M={M} K={K} N={N}")


@pytest.mark.parametrize("name", ["decode1", "decode8", "decode32", "decode64"])
def test_nv_linear_decode(name):
    """The decode workloads (K = N = 4096, no RMSNorm): every output."""
    print(f"nv linear {name}", flush=True)
    inp = synth.layer_inputs(name, seed=0)
    act, wt, y = nv_layer(inp["x"], inp["gamma"], inp["w"])
    ref = O.prepare_nv(inp["x"], inp["gamma"], inp["eps"])
    wc, ws, gw = O.pack_weight_nv(inp["w"])
    yr, b = O.linear_nv(ref, wc, ws, gw)
    assert_linear_close(y.cpu().numpy(), yr, b, name)


def test_nv_linear_bf16_out_and_zero():
    import torch
    print("nv linear bf16 / zero", flush=True)
    rng = np.random.default_rng(5)
    x = synth.outlier_activations(rng, 8, 512)
    w = synth.linear_weight(rng, 64, 512)
    _, _, y32 = nv_layer(x, None, w)
    _, _, y16 = nv_layer(x, None, w, out_dtype=sq.OUT_BF16)
    want = y32.to(torch.bfloat16)
    assert torch.equal(y16.view(torch.int16), want.view(torch.int16))
    _, _, yz = nv_layer(np.zeros_like(x), None, w)
    assert torch.count_nonzero(yz).item() == 0
