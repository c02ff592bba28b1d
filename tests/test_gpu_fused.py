"""GPU parity of the one-launch small-M layer (sharq_linear_fused): identical
bit for bit to sharq_prepare + sharq_linear, and within 1e-5 * sum|terms| +
1e-6 of the float64 oracle."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, dev_bf16

pytestmark = pytest.mark.gpu


# M * K / 32 <= 1024 takes the register-resident path; (16, 4096) and (12, 8192) the other
@pytest.mark.parametrize("M,K,N,norm", [(1, 4096, 4096, False), (8, 4096, 4096, False), (16, 2048, 1536, True),
                                        (5, 96, 53, True), (3, 8192, 200, True), (13, 1376, 100, False),
                                        (1, 4096, 4096, True), (16, 4096, 512, True), (12, 8192, 300, False),
                                        (9, 4096, 100, True)])
def test_fused_layer(M, K, N, norm):
    import torch
    print(f"fused M={M} K={K} N={N} norm={norm}", flush=True)
    rng = np.random.default_rng(M * 11 + K + N)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    xd, gd = dev_bf16(x), (dev_bf16(g) if norm else None)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    y1 = sq.sharq_linear_fused(xd, wt, gd, 1e-5)
    y2 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5), wt)
    yb = sq.sharq_linear_fused(xd, wt, gd, 1e-5, out_dtype=sq.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), float((y1 - y2).abs().max())
    assert torch.equal(yb.view(torch.int16), y1.to(torch.bfloat16).view(torch.int16))
    ref = O.prepare(x, g, 1e-5)
    wc, ws = O.pack_weight(w)
    yr, b = O.linear(ref, wc, ws)
    assert_linear_close(y1.cpu().numpy(), yr, b, f"fused M={M}")


def test_fused_decode_workloads():
    import torch
    for name in ("decode1", "decode8"):
        print(f"fused {name}", flush=True)
        inp = synth.layer_inputs(name, seed=1)
        wt = sq.sharq_pack_weight(dev_bf16(inp["w"]))
        y = sq.sharq_linear_fused(dev_bf16(inp["x"]), wt)
        torch.cuda.synchronize()
        ref = O.prepare(inp["x"], None, inp["eps"])
        wc, ws = O.pack_weight(inp["w"])
        yr, b = O.linear(ref, wc, ws)
        assert_linear_close(y.cpu().numpy(), yr, b, name)


@pytest.mark.parametrize("M,K,N,norm", [(1, 4096, 4096, False), (1, 4096, 4096, True), (5, 96, 53, True),
                                        (16, 2048, 300, False), (8, 8192, 64, True), (3, 1376, 100, False)])
def test_fused_layer_nvfp4(M, K, N, norm):
    """NVFP4-style in one launch: identical to sharq_prepare(fmt NVFP4) +
    sharq_linear, and within tolerance of the float64 oracle."""
    import torch
    print(f"fused nvfp4 M={M} K={K} N={N} norm={norm}", flush=True)
    rng = np.random.default_rng(M * 7 + K + N + 1)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    xd, gd = dev_bf16(x), (dev_bf16(g) if norm else None)
    wt = sq.sharq_pack_weight(dev_bf16(w), fmt=sq.FMT_NVFP4)
    y1 = sq.sharq_linear_fused(xd, wt, gd, 1e-5)
    y2 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5, fmt=sq.FMT_NVFP4), wt)
    yb = sq.sharq_linear_fused(xd, wt, gd, 1e-5, out_dtype=sq.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), float((y1 - y2).abs().max())
    assert torch.equal(yb.view(torch.int16), y1.to(torch.bfloat16).view(torch.int16))
    ref = O.prepare_nv(x, g, 1e-5)
    wc, ws, wg = O.pack_weight_nv(w)
    yr, b = O.linear_nv(ref, wc, ws, wg)
    assert_linear_close(y1.cpu().numpy(), yr, b, f"fused nvfp4 M={M}")
