"""GPU parity of the grouped gate/up layer whose SwiGLU epilogue prepares the
down projection's activation (sharq_linear_grouped_swiglu_prep): byte for byte
the activation sharq_prepare writes for the routed rows of H, where expert e's
rows of H are sharq_linear_swiglu of its routed rows with its own interleaved
gate/up weight -- every tiled array, the padding rows of the last block
included -- and, through that, the oracle's preparation of H.  The down
projection on the fused activation equals the down projection on that
reference activation."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_prep_equal, dev_bf16, untile_act

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _reference_h(x, wg, wu, experts, seg, token):
    """Routed rows of H, expert by expert through the dense layer: the rows of
    expert e are its routed source rows (zero rows for indices out of range)."""
    import torch
    F, K = wg.shape[0] // experts, x.shape[1]
    hs = []
    for e in range(experts):
        lo, hi = int(seg[e]), int(seg[e + 1])
        if hi == lo:
            continue
        idx = token[lo:hi].astype(np.int64)
        ok = (idx >= 0) & (idx < x.shape[0])
        xe = np.zeros((hi - lo, K), dtype=x.dtype)
        xe[ok] = x[idx[ok]]
        act = sq.sharq_prepare(dev_bf16(xe), None)
        w = sq.sharq_pack_weight(sq.interleave_gate_up(dev_bf16(wg[e * F:(e + 1) * F]), dev_bf16(wu[e * F:(e + 1) * F])))
        hs.append(sq.sharq_linear_swiglu(act, w))
    return torch.cat(hs) if hs else torch.empty(0, F, dtype=torch.bfloat16, device="cuda")


def _case(seed, tokens, experts, top_k, K, F, holes=False):
    rng = np.random.default_rng(seed)
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    if holes:                                           # routed rows that read as zero input
        token = token.copy()
        token[3], token[len(token) // 2] = tokens + 1000, -1
    x = synth.outlier_activations(rng, tokens, K)
    wg = np.concatenate([synth.linear_weight(rng, F, K) for _ in range(experts)])
    wu = np.concatenate([synth.linear_weight(rng, F, K) for _ in range(experts)])
    return x, wg, wu, token, seg


def _fused(x, wg, wu, experts, seg, token, in_order=False):
    import torch
    if in_order:                                        # rows already in expert order: no row index
        act = sq.sharq_prepare(dev_bf16(x[token]), None)
        ri = None
    else:
        act = sq.sharq_prepare(dev_bf16(x), None)
        ri = _dev(token.astype(np.int32), torch.int32)
    w = sq.sharq_pack_weight(sq.interleave_gate_up(dev_bf16(wg), dev_bf16(wu), experts=experts))
    return sq.sharq_linear_grouped_swiglu_prep(act, w, _dev(seg, torch.int64), experts, row_index=ri,
                                               rows=int(seg[-1]))


def _assert_same_act(a, b, label):
    import torch
    torch.cuda.synchronize()
    assert (a.M, a.K, a.n, a.m, a.fmt) == (b.M, b.K, b.n, b.m, b.fmt), label
    for f in sq.SharqAct.FIELDS:
        u, v = getattr(a, f), getattr(b, f)
        assert u.numel() == v.numel() and torch.equal(u, v), f"{label}: {f}"


@pytest.mark.parametrize("seed,tokens,experts,top_k,K,F,holes,in_order", [
    (0, 203, 6, 2, 256, 128, True, False),      # 406 routed rows (a ragged last block), zero-input rows
    (1, 512, 4, 2, 512, 256, False, False),     # experts spanning several 128-row tiles
    (2, 203, 6, 2, 256, 128, False, True),      # rows already in expert order
    (3, 64, 16, 1, 128, 384, False, False),     # empty experts, four N tiles per expert
    (4, 100, 5, 2, 160, 128, True, False),      # K = 160: a partial last K tile
])
def test_grouped_swiglu_prep_equals_per_expert_layers(seed, tokens, experts, top_k, K, F, holes, in_order):
    print(f"grouped swiglu_prep seed={seed} tokens={tokens} E={experts} K={K} F={F}", flush=True)
    x, wg, wu, token, seg = _case(seed, tokens, experts, top_k, K, F, holes)
    nxt = _fused(x, wg, wu, experts, seg, token, in_order)
    ref = sq.sharq_prepare(_reference_h(x, wg, wu, experts, seg, token), None)
    _assert_same_act(nxt, ref, f"seed {seed}")


def test_grouped_swiglu_prep_matches_oracle_prepare():
    import torch
    x, wg, wu, token, seg = _case(5, 150, 5, 2, 256, 128, holes=True)
    nxt = _fused(x, wg, wu, 5, seg, token)
    h = _reference_h(x, wg, wu, 5, seg, token)
    torch.cuda.synchronize()
    rows = int(seg[-1])
    hb = h.view(torch.int16).cpu().numpy().astype(np.uint16)
    assert_prep_equal(untile_act(nxt.host(), rows, 128), O.prepare(hb, None, 1e-5), "grouped swiglu_prep")


def test_grouped_swiglu_prep_qwen_shape_and_down():
    """The Qwen3-30B-A3B expert MLP shape as the benchmark runs it (4096 tokens,
    top-8 of 128 experts, K = 2048, F = 768); then the down projection (K = 768,
    N_e = 2048) on the fused activation equals it on the reference one."""
    import torch
    print("grouped swiglu_prep qwen shape", flush=True)
    x, wg, wu, token, seg = _case(11, 4096, 128, 8, 2048, 768)
    nxt = _fused(x, wg, wu, 128, seg, token)
    ref = sq.sharq_prepare(_reference_h(x, wg, wu, 128, seg, token), None)
    _assert_same_act(nxt, ref, "qwen")
    rng = np.random.default_rng(12)
    wd = sq.sharq_pack_weight(dev_bf16(np.concatenate([synth.linear_weight(rng, 2048, 768) for _ in range(128)])))
    seg_d = _dev(seg, torch.int64)
    y1 = sq.sharq_linear_grouped(nxt, wd, seg_d, 128)
    y2 = sq.sharq_linear_grouped(ref, wd, seg_d, 128)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
