"""GPU parity past 2 GiB of prepared codes.  An activation of 2^20 + 37 rows x
4096 (each code array 2.15 GB) no longer fits the tiled GEMM's 31-bit buffer
offsets, so the layer runs the split-K kernel with two row blocks per workgroup
and 64-bit addressing; the preparation addresses its tiles with 64-bit indices
too.  The rows repeat with period 4099 (not a power of two: a wrapped or
truncated address would land on a different row).  Sampled rows -- the first
ones, random ones and every row whose tiles lie past the 2^31-byte boundary --
are recomputed by the oracle: their prepared bytes, read straight out of the
tiled layout on the device, byte for byte, and their outputs within the GEMM
tolerance."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, assert_prep_equal, dev_bf16

pytestmark = pytest.mark.gpu

M, K, N, PERIOD = (1 << 20) + 37, 4096, 48, 4099


def _rows_of_tiled(act, rows):
    """The sampled rows' prepared arrays in the oracle's row-major form, gathered
    on the device from the tiled layout (16 rows x 128 K per tile, lane = row % 16
    + 16 * chunk; scale bytes K-tile major)."""
    import torch
    RB, KT = (act.M + 15) // 16, K // 128
    r = torch.as_tensor(rows, device="cuda", dtype=torch.int64)
    rb, r16 = (r // 16)[:, None, None], (r % 16)[:, None, None]
    kt = torch.arange(KT, device="cuda")[None, :, None]
    c = torch.arange(4, device="cuda")[None, None, :]
    lane = c * 16 + r16
    tile = rb * KT + kt
    b16 = torch.arange(16, device="cuda")
    codes_idx = ((tile * 1024 + lane * 16)[..., None] + b16).reshape(len(rows), -1)
    meta_idx = ((tile * 256 + lane * 4)[..., None] + torch.arange(4, device="cuda")).reshape(len(rows), -1)
    scale_idx = ((kt * RB + rb) * 64 + lane).reshape(len(rows), -1)
    out = {}
    for f, idx in (("s_codes", codes_idx), ("r_codes", codes_idx), ("s_meta", meta_idx),
                   ("s_scales", scale_idx), ("r_scales", scale_idx)):
        out[f] = getattr(act, f).reshape(-1)[idx.reshape(-1)].reshape(idx.shape).cpu().numpy()
    return out


def test_layer_past_31_bit_offsets():
    import torch
    print(f"linear past 2 GiB of codes: M={M} K={K} N={N}", flush=True)
    rng = np.random.default_rng(20)
    base = synth.outlier_activations(rng, PERIOD, K)
    g = synth.norm_weight(rng, K)
    w = synth.linear_weight(rng, N, K)
    RB, KT = (M + 15) // 16, K // 128
    assert RB * KT * 1024 > 0x7FFFFFFF                     # past the tiled kernel's offsets
    x = dev_bf16(base).index_select(0, torch.arange(M, device="cuda") % PERIOD)
    act = sq.sharq_prepare(x, dev_bf16(g), 1e-5)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    y = sq.sharq_linear(act, wt)
    torch.cuda.synchronize()
    del x
    # every row whose tiles start past 2^31 bytes, the first rows and random ones
    first_past = (0x80000000 // (KT * 1024)) * 16
    rows = np.unique(np.concatenate([np.arange(6), np.arange(first_past - 3, M),
                                     rng.choice(M, 16, replace=False)]))
    assert rows.max() == M - 1 and len(rows) > 50
    ref = O.prepare(base[rows % PERIOD], g, 1e-5)
    assert_prep_equal(_rows_of_tiled(act, rows), ref, "large")
    wc, ws = O.pack_weight(w)
    yr, b = O.linear(ref, wc, ws)
    yg = y[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    assert_linear_close(yg, yr, b, "large")
    del act, y
    torch.cuda.empty_cache()
