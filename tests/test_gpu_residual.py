"""GPU parity of the layer with the residual add in its epilogue
(sharq_linear_residual): bit for bit sharq_linear (fp32) followed by
sharq_add_bf16_f32, on the split-K (small M) and tiled kernels, ragged and
strided shapes, the plain FP4 pattern and in place; and against the oracle."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _layer(M, K, N, norm, n=2, seed=0):
    rng = np.random.default_rng(seed + M + K + N)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    res = synth.outlier_activations(rng, M, N)
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(g) if norm else None, 1e-5, n=n, m=4)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    return x, g, w, res, act, wt


@pytest.mark.parametrize("M,K,N,norm,n", [(37, 96, 53, True, 2), (5, 1376, 100, False, 2), (130, 768, 200, False, 2),
                                          (300, 2048, 1536, True, 2), (2048, 4096, 4096, False, 2),
                                          (257, 512, 384, True, 0),
                                          # 256 x 192 tiles: whole and ragged M tiles
                                          (2048, 256, 6144, False, 2), (2000, 512, 6144, True, 2),
                                          # split-K (M <= 64): one, two and four column blocks per
                                          # workgroup, partial row blocks
                                          (1, 4096, 4096, False, 2), (32, 1024, 4096, False, 2),
                                          (63, 1056, 2025, True, 2), (64, 512, 4100, False, 2)])
def test_residual_layer_equals_two_calls(M, K, N, norm, n):
    import torch
    print(f"residual M={M} K={K} N={N} n={n}", flush=True)
    x, g, w, res, act, wt = _layer(M, K, N, norm, n)
    r = dev_bf16(res)
    y = sq.sharq_linear_residual(act, wt, r)
    ref = sq.sharq_add_bf16_f32(r, sq.sharq_linear(act, wt))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_residual_layer_strided_and_in_place():
    import torch
    M, K, N = 96, 512, 200
    x, g, w, res, act, wt = _layer(M, K, N, True)
    wide = torch.zeros(M, N + 3, dtype=torch.bfloat16, device="cuda")
    wide[:, :N] = dev_bf16(res)
    r = wide[:, :N]                                   # row stride N + 3: element-wise stores
    ref = sq.sharq_add_bf16_f32(dev_bf16(res), sq.sharq_linear(act, wt))
    y = sq.sharq_linear_residual(act, wt, r)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    inplace = dev_bf16(res).clone()
    sq.sharq_linear_residual(act, wt, inplace, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace.view(torch.int16), ref.view(torch.int16))


def test_residual_layer_against_oracle():
    import torch
    M, K, N = 37, 256, 48
    x, g, w, res, act, wt = _layer(M, K, N, True)
    y = sq.sharq_linear_residual(act, wt, dev_bf16(res))
    torch.cuda.synchronize()
    got = (y.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ref = O.prepare(x, g, 1e-5)
    wc, ws = O.pack_weight(w)
    yr, b = O.linear(ref, wc, ws)
    exact = O.widen_bf16(res).astype(np.float64) + yr
    # the layer tolerance, then the binary32 add and the bf16 rounding (half an ulp of 8 bits)
    bound = 1e-5 * b + 1e-6 + np.abs(exact) * (2.0 ** -8 + 2.0 ** -23) + 1e-30
    assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)
