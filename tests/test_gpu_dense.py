"""GPU parity of the plain FP4 linear (pattern 0:4: no backbone, MXFP4 of the
normalised row, the dense GEMM path alone) -- the dense FP4 baseline SharQ is
compared against.  Prep bytes exact against the oracle, GEMM within
1e-5 * sum|terms| + 1e-6."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, dev_bf16, untile_dense, untile_scales

pytestmark = pytest.mark.gpu


def dense_layer(x, gamma, w, eps=1e-5):
    import torch
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(gamma) if gamma is not None else None, eps, n=0, m=4)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    y = sq.sharq_linear(act, wt)
    torch.cuda.synchronize()
    return act, y


def check_prep(act, ref, M, K, label):
    assert act.s_codes.numel() == 0 and act.s_meta.numel() == 0 and act.s_scales.numel() == 0
    codes = untile_dense(act.r_codes.cpu().numpy(), M, K, "r_codes")
    scales = untile_scales(act.r_scales.cpu().numpy(), M, K, "r_scales")
    assert np.array_equal(scales, ref["r_scales"]), label
    assert np.array_equal(codes, ref["r_codes"]), label


@pytest.mark.parametrize("M,K,N,norm", [(37, 96, 53, True), (130, 768, 200, False), (5, 1376, 100, False),
                                        (256, 256, 272, True), (1, 4096, 4096, False), (64, 4096, 4096, False),
                                        (300, 16384, 64, True), (63, 1056, 2025, False), (64, 1056, 4100, True)])
def test_dense_linear_full(M, K, N, norm):
    print(f"dense M={M} K={K} N={N} norm={norm}", flush=True)
    rng = np.random.default_rng(M * 7 + K + N)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    w = synth.linear_weight(rng, N, K)
    act, y = dense_layer(x, g, w)
    ref = O.prepare_dense(x, g, 1e-5)
    check_prep(act, ref, M, K, f"M={M} K={K}")
    wc, ws = O.pack_weight(w)
    yr, b = O.linear_dense(ref, wc, ws)
    assert_linear_close(y.cpu().numpy(), yr, b, f"dense M={M} K={K} N={N}")


def test_dense_qkv_sampled():
    """Full QKV size (2048 x 4096 -> 6144, RMSNorm) on the tiled kernel; the
    oracle recomputes sampled rows."""
    print("dense qkv", flush=True)
    inp = synth.layer_inputs("qkv", seed=0)
    act, y = dense_layer(inp["x"], inp["gamma"], inp["w"])
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(2044, 2048), rng.choice(2048, 16, replace=False)]))
    ref = O.prepare_dense(inp["x"][rows], inp["gamma"], inp["eps"])
    wc, ws = O.pack_weight(inp["w"])
    yr, b = O.linear_dense(ref, wc, ws)
    assert_linear_close(y.cpu().numpy()[rows], yr, b, "dense qkv")
