"""GPU parity of the fusion ablations: the unfused RMSNorm (bf16 output bit-exact
against the oracle, and the preparation of that bf16 row bit-exact), and the
unfused epilogue (each GEMM path alone, then the add kernel) within
1e-5 * sum|terms| + 1e-6 of the float64 oracle."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, assert_prep_equal, dev_bf16, untile_act

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 4096), (37, 96), (130, 768), (5, 32768), (2048, 4096)])
def test_unfused_rmsnorm_bit_exact(M, K):
    import torch
    print(f"rmsnorm M={M} K={K}", flush=True)
    rng = np.random.default_rng(M + K)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K)
    y = sq.sharq_rmsnorm(dev_bf16(x), dev_bf16(g), 1e-5)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.rmsnorm_bf16(x, g, 1e-5)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4])
    if M <= 130:
        # the unfused preparation: bf16 row, no gamma
        act = sq.sharq_prepare(y, None, 1e-5)
        torch.cuda.synchronize()
        assert_prep_equal(untile_act(act.host(), M, K), O.prepare(want, None, 1e-5), f"unfused M={M}")


@pytest.mark.parametrize("M,K,N", [(37, 96, 53), (130, 768, 200), (1, 4096, 4096), (256, 2048, 384)])
def test_unfused_epilogue(M, K, N):
    import torch
    print(f"unfused epilogue M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M * 3 + K + N)
    x = synth.outlier_activations(rng, M, K)
    g = synth.norm_weight(rng, K)
    w = synth.linear_weight(rng, N, K)
    act = sq.sharq_prepare(dev_bf16(x), dev_bf16(g), 1e-5)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    ys = sq.sharq_linear(sq.path_act(act, "backbone"), wt)
    yr = sq.sharq_linear(sq.path_act(act, "residual"), wt)
    y = sq.sharq_add_f32(ys, yr)
    torch.cuda.synchronize()
    ref = O.prepare(x, g, 1e-5)
    wc, ws = O.pack_weight(w)
    rs, rr, b = O.linear_paths(ref, wc, ws)
    assert_linear_close(ys.cpu().numpy(), rs, b, f"backbone path M={M}")
    assert_linear_close(yr.cpu().numpy(), rr, b, f"residual path M={M}")
    assert_linear_close(y.cpu().numpy(), rs + rr, b, f"unfused M={M}")
    # the add kernel is exact binary32 addition
    assert torch.equal(y, ys + yr)


@pytest.mark.parametrize("n,off", [(1 << 20, 0), (1000003, 0), (4099, 1)])
def test_residual_add_bit_exact(n, off):
    import torch
    print(f"residual add n={n} off={off}", flush=True)
    rng = np.random.default_rng(n)
    x = synth.bf16_bits_from_f32(rng.standard_normal(n + off).astype(np.float32) * 4)
    y = (rng.standard_normal(n + off) * 3).astype(np.float32)
    xd = dev_bf16(x)[off:]
    yd = torch.from_numpy(y).cuda()[off:]
    out = sq.sharq_add_bf16_f32(xd, yd)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, O.residual_add_bf16(x[off:], y[off:]))
