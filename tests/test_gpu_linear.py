"""GPU parity of the dual FP4 GEMM: |y_gpu - y_ref| <= 1e-5 * sum|terms| + 1e-6
elementwise against the float64 oracle, on full outputs for small shapes and on
sampled rows/columns of the full-size workloads."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, assert_prep_equal, dev_bf16, untile_act

pytestmark = pytest.mark.gpu


def gpu_layer(x, gamma, w, eps=1e-5, out_dtype=sq.OUT_F32):
    import torch
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(gamma) if gamma is not None else None, eps)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    y = sq.sharq_linear(act, wt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return act, wt, y


def test_linear_tiny_full():
    print("linear tiny", flush=True)
    inp = synth.layer_inputs("tiny", seed=0)
    act, wt, y = gpu_layer(inp["x"], inp["gamma"], inp["w"])
    ref = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    assert_prep_equal(untile_act(act.host(), 16, 256), ref, "tiny")
    wc, ws = O.pack_weight(inp["w"])
    yr, b = O.linear(ref, wc, ws)
    assert_linear_close(y.cpu().numpy(), yr, b, "tiny")


@pytest.mark.parametrize("M,K,N,norm", [(37, 96, 53, True), (1, 4096, 4096, False), (130, 768, 200, False),
                                        (64, 4096, 4096, False), (17, 2048, 1536, False), (256, 256, 272, True),
                                        (5, 1376, 100, False), (3, 14336, 64, False), (49, 640, 48, True),
                                        (63, 1056, 2025, False), (64, 1056, 4100, True)])
def test_linear_ragged_full(M, K, N, norm):
    print(f"linear M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M + K + N)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    act, wt, y = gpu_layer(x, g, w)
    ref = O.prepare(x, g, 1e-5)
    wc, ws = O.pack_weight(w)
    yr, b = O.linear(ref, wc, ws)
    assert_linear_close(y.cpu().numpy(), yr, b, f"M={M} K={K} N={N}")


@pytest.mark.parametrize("name", ["decode1", "decode8", "decode32", "decode64"])
def test_linear_decode_full(name):
    """Decode shapes (M in {1, 8, 32, 64}, K = N = 4096): every output against the oracle."""
    print(f"linear {name}", flush=True)
    inp = synth.layer_inputs(name, seed=0)
    act, wt, y = gpu_layer(inp["x"], inp["gamma"], inp["w"])
    ref = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(inp["w"])
    yr, b = O.linear(ref, wc, ws)
    assert_linear_close(y.cpu().numpy(), yr, b, name)


def _sample_rows(M, rng, n=24):
    return np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), rng.choice(M, n, replace=False)]))


@pytest.mark.parametrize("name,ncols", [("qkv", None), ("down", None), ("gateup", 2048)])
def test_linear_workloads_sampled(name, ncols):
    """Full-size GEMM on the GPU; the oracle recomputes sampled rows (and, for the
    widest layer, sampled columns) one by one."""
    print(f"linear {name}", flush=True)
    inp = synth.layer_inputs(name, seed=0)
    act, wt, y = gpu_layer(inp["x"], inp["gamma"], inp["w"])
    rng = np.random.default_rng(1)
    rows = _sample_rows(inp["M"], rng)
    cols = np.arange(inp["N"]) if ncols is None else np.unique(np.concatenate(
        [np.arange(16), np.arange(inp["N"] - 16, inp["N"]), rng.choice(inp["N"], ncols, replace=False)]))
    ref = O.prepare(inp["x"][rows], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(inp["w"][cols])
    yr, b = O.linear(ref, wc, ws)
    yg = y.cpu().numpy()[np.ix_(rows, cols)]
    assert_linear_close(yg, yr, b, name)


def test_linear_bf16_output():
    inp = synth.layer_inputs("tiny", seed=0)
    _, _, y = gpu_layer(inp["x"], inp["gamma"], inp["w"], out_dtype=sq.OUT_BF16)
    ref = O.prepare(inp["x"], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(inp["w"])
    yr, b = O.linear(ref, wc, ws)
    import torch
    yg = y.float().cpu().numpy()
    half_ulp = np.abs(yr) * 2.0 ** -8
    assert_linear_close(yg, yr, b, "bf16 out", extra=half_ulp)


@pytest.mark.parametrize("M", [256, 48])
def test_linear_deterministic_and_strided_output(M):
    import torch
    inp = synth.layer_inputs("qkv", seed=1, M=M)
    act = sq.sharq_prepare(dev_bf16(inp["x"]), dev_bf16(inp["gamma"]))
    wt = sq.sharq_pack_weight(dev_bf16(inp["w"]))
    y1 = sq.sharq_linear(act, wt)
    big = torch.full((M, inp["N"] + 64), 7.0, device="cuda")
    y2 = sq.sharq_linear(act, wt, out=big[:, 32:32 + inp["N"]])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.all(big[:, :32] == 7.0) and torch.all(big[:, 32 + inp["N"]:] == 7.0)


@pytest.mark.parametrize("M,K,N", [(512, 512, 384), (512, 1024, 6144), (300, 512, 200), (2048, 256, 4096),
                                   # 256 x 192 tiles (fewer waves of workgroups than 128 x 256 ones): whole
                                   # tiles in rounds of two 16-row blocks, and a ragged last M tile
                                   (2048, 512, 6144), (2000, 256, 6144),
                                   # split-K (M <= 64): one, two and four column blocks per workgroup
                                   (1, 4096, 4096), (32, 1024, 4096), (63, 1056, 2025), (64, 512, 4100)])
def test_linear_tiled_bf16_equals_rounded_fp32(M, K, N):
    """The bf16 output (tiled kernel: staged through LDS for whole tiles,
    element-wise at ragged edges; split-K kernel: element-wise) is the fp32
    output rounded to nearest even."""
    import torch
    print(f"tiled bf16 M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M + K + N + 7)
    x = synth.outlier_activations(rng, M, K)
    w = synth.linear_weight(rng, N, K)
    act = sq.sharq_prepare(dev_bf16(x), None, 1e-5)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    y32 = sq.sharq_linear(act, wt)
    y16 = sq.sharq_linear(act, wt, out_dtype=sq.OUT_BF16)
    wide = torch.zeros(M, N + 8, dtype=torch.bfloat16, device="cuda")
    sq.sharq_linear(act, wt, out=wide[:, :N], out_dtype=sq.OUT_BF16)   # row stride N + 8
    torch.cuda.synchronize()
    ref = y32.to(torch.bfloat16).view(torch.int16)
    assert torch.equal(y16.view(torch.int16), ref)
    assert torch.equal(wide[:, :N].contiguous().view(torch.int16), ref)
