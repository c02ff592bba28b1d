"""The grouped expert layer's allocation-free entry point
(sharq_linear_grouped_noalloc, for callers that cannot allocate) through the C
ABI: its outputs equal those of sharq_linear_grouped with a caller workspace,
bit for bit (same kernels, same inputs), on consecutive calls that share the
library's scratch -- the second call smaller than the first -- with routed
token rows (gathered into the scratch) and rows already in expert order."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _layer(tokens, E, top_k, K, Ne, seed):
    import torch
    rng = np.random.default_rng(seed)
    expert, token, seg = synth.zipf_router(rng, tokens, E, top_k)
    x_tok = synth.outlier_activations(rng, tokens, K)
    x_rows = synth.outlier_activations(rng, tokens * top_k, K)
    w = np.concatenate([synth.linear_weight(rng, Ne, K) for _ in range(E)])
    act_tok = sq.sharq_prepare(dev_bf16(x_tok), None)
    act_rows = sq.sharq_prepare(dev_bf16(x_rows), None)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    seg_d = torch.from_numpy(seg).cuda()
    ri = torch.from_numpy(token.astype(np.int32)).cuda()
    return act_tok, act_rows, wt, seg_d, ri, tokens * top_k


@pytest.mark.parametrize("out_dtype", [sq.OUT_F32, sq.OUT_BF16])
def test_noalloc_equals_workspace_entry_point(out_dtype):
    import torch
    # the first call larger than the second: the scratch keeps the first call's
    # contents when the second runs
    for tokens, E, top_k, K, Ne, seed in [(512, 16, 4, 1024, 128, 0), (96, 8, 2, 512, 64, 1)]:
        print(f"noalloc tokens={tokens} E={E} top_k={top_k} K={K} N_e={Ne}", flush=True)
        act_tok, act_rows, wt, seg, ri, rows = _layer(tokens, E, top_k, K, Ne, seed)
        need = sq.grouped_workspace_bytes(rows, E, K)
        assert need <= sq.noalloc_scratch_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref_g = sq.sharq_linear_grouped(act_tok, wt, seg, E, row_index=ri, rows=rows, out_dtype=out_dtype, workspace=ws)
        ref_s = sq.sharq_linear_grouped(act_rows, wt, seg, E, out_dtype=out_dtype, workspace=ws)
        got_g = sq.sharq_linear_grouped_noalloc(act_tok, wt, seg, E, row_index=ri, rows=rows, out_dtype=out_dtype)
        got_s = sq.sharq_linear_grouped_noalloc(act_rows, wt, seg, E, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(got_g.view(torch.int32 if out_dtype == sq.OUT_F32 else torch.int16),
                           ref_g.view(torch.int32 if out_dtype == sq.OUT_F32 else torch.int16))
        assert torch.equal(got_s.view(torch.int32 if out_dtype == sq.OUT_F32 else torch.int16),
                           ref_s.view(torch.int32 if out_dtype == sq.OUT_F32 else torch.int16))


def test_noalloc_rejects_a_layer_past_its_scratch():
    import torch
    act_tok, act_rows, wt, seg, ri, rows = _layer(64, 4, 2, 256, 32, 2)
    big = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")   # 2^20 routed rows: past 32 MiB of workspace
    assert sq.grouped_workspace_bytes(big.numel(), 4, 256) > sq.noalloc_scratch_bytes()
    with pytest.raises(sq.SharqError) as e:
        sq.sharq_linear_grouped_noalloc(act_tok, wt, seg, 4, row_index=big)
    assert e.value.status == 3
