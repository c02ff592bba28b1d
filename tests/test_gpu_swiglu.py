"""GPU parity of the gate/up layer with the SwiGLU epilogue: H = bf16(SiLU(gate)
* up) against the float64 oracle, within the GEMM tolerance carried through
SiLU and the product plus the bf16 rounding (swiglu_bound)."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,F,norm", [(37, 96, 32, True), (130, 768, 96, False), (256, 512, 64, True),
                                        (300, 2048, 1536, True), (5, 1376, 48, False)])
def test_swiglu_layer(M, K, F, norm):
    import torch
    print(f"swiglu M={M} K={K} F={F} norm={norm}", flush=True)
    rng = np.random.default_rng(M + K + F)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    wg = synth.linear_weight(rng, F, K)
    wu = synth.linear_weight(rng, F, K)
    wgu = O.interleave_gate_up(wg, wu)
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(g) if norm else None, 1e-5)
    wt = sq.sharq_pack_weight(dev_bf16(wgu))
    h = sq.sharq_linear_swiglu(act, wt)
    torch.cuda.synchronize()
    got = h.float().cpu().numpy().astype(np.float64)
    ref = O.prepare(x, g, 1e-5)
    wc, ws = O.pack_weight(wgu)
    hr, bg, bu, gt, up = O.linear_swiglu(ref, wc, ws)
    bound = O.swiglu_bound(gt, up, bg, bu)
    bad = np.argwhere(np.abs(got - hr) > bound)
    assert bad.size == 0, (len(bad), [(float(got[i, j]), float(hr[i, j]), float(bound[i, j])) for i, j in bad[:4]])


def test_swiglu_interleave_matches_torch_helper():
    import torch
    rng = np.random.default_rng(1)
    wg = synth.linear_weight(rng, 48, 64)
    wu = synth.linear_weight(rng, 48, 64)
    a = sq.interleave_gate_up(dev_bf16(wg), dev_bf16(wu)).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a, O.interleave_gate_up(wg, wu))


def test_swiglu_gateup_sampled():
    """Full gate/up size (2048 x 4096 -> 2 x 14336, RMSNorm) on the kernel the
    decoder layer times; the oracle recomputes sampled rows and h columns from
    the separate gate and up weights."""
    import torch
    print("swiglu gate/up sampled", flush=True)
    M, K, F = 2048, 4096, 14336
    inp = synth.layer_inputs("qkv", seed=5, with_weight=False)
    rng = np.random.default_rng(6)
    wg = synth.linear_weight(rng, F, K)
    wu = synth.linear_weight(rng, F, K)
    act = sq.sharq_prepare(dev_bf16(inp["x"]), dev_bf16(inp["gamma"]), inp["eps"])
    wt = sq.sharq_pack_weight(sq.interleave_gate_up(dev_bf16(wg), dev_bf16(wu)))
    h = sq.sharq_linear_swiglu(act, wt)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), rng.choice(M, 24, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(16), np.arange(F - 16, F), rng.choice(F, 512, replace=False)]))
    got = h.float().cpu().numpy().astype(np.float64)[np.ix_(rows, cols)]
    ref = O.prepare(inp["x"][rows], inp["gamma"], inp["eps"])
    gc, gs = O.pack_weight(wg[cols])
    uc, us = O.pack_weight(wu[cols])
    gt, bg = O.linear(ref, gc, gs)
    up, bu = O.linear(ref, uc, us)
    hr = O.silu(gt) * up
    bound = O.swiglu_bound(gt, up, bg, bu)
    bad = np.argwhere(np.abs(got - hr) > bound)
    assert bad.size == 0, (len(bad), [(float(got[i, j]), float(hr[i, j]), float(bound[i, j])) for i, j in bad[:4]])
