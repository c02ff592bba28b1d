"""GPU parity of the gate/up layer whose SwiGLU epilogue prepares the down
projection's activation (sharq_linear_swiglu_prep): byte for byte the
activation sharq_prepare writes for the H that sharq_linear_swiglu stores --
every tiled array, padding rows and the ragged last gate/up tile included --
and, through that, the oracle's preparation of H."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_prep_equal, dev_bf16, untile_act

pytestmark = pytest.mark.gpu


def _gate_up(M, K, F, norm, seed=0):
    rng = np.random.default_rng(seed + M + K + F)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K) if norm else None
    wg, wu = synth.linear_weight(rng, F, K), synth.linear_weight(rng, F, K)
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(g) if norm else None, 1e-5)
    wt = sq.sharq_pack_weight(sq.interleave_gate_up(dev_bf16(wg), dev_bf16(wu)))
    return act, wt


@pytest.mark.parametrize("M,K,F,norm", [(37, 96, 128, True), (130, 768, 256, False), (300, 2048, 1536, True),
                                        (16, 512, 384, False), (2048, 4096, 14336, True)])
def test_swiglu_prep_equals_store_then_prepare(M, K, F, norm):
    import torch
    print(f"swiglu_prep M={M} K={K} F={F} norm={norm}", flush=True)
    act, wt = _gate_up(M, K, F, norm)
    nxt = sq.sharq_linear_swiglu_prep(act, wt)
    ref = sq.sharq_prepare(sq.sharq_linear_swiglu(act, wt), None, 1e-5)
    torch.cuda.synchronize()
    for f in sq.SharqAct.FIELDS:
        a, b = getattr(nxt, f), getattr(ref, f)
        assert a.numel() == b.numel() and torch.equal(a, b), f


def test_swiglu_prep_matches_oracle_prepare():
    import torch
    M, K, F = 40, 256, 128
    act, wt = _gate_up(M, K, F, True, seed=3)
    nxt = sq.sharq_linear_swiglu_prep(act, wt)
    h = sq.sharq_linear_swiglu(act, wt)
    torch.cuda.synchronize()
    hb = h.view(torch.int16).cpu().numpy().astype(np.uint16)
    assert_prep_equal(untile_act(nxt.host(), M, F), O.prepare(hb, None, 1e-5), "swiglu_prep")
