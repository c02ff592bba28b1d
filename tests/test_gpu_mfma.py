"""GPU probe of the block-scaled FP4 MFMA as the GEMM kernels issue it
(sharq_check_mfma_fp4): one 16 x 16 x 128 product per block on operands in the
tiled lane order, against its definition d[m][n] = sum over k of deq(A)[m][k] *
deq(B)[n][k], with deq the oracle's MX dequantisation (float64).  One-hot blocks
pin the operand, scale and accumulator lane layouts bit for bit (one nonzero
product per block, every (m, n), every 32-element chunk and every position in
it; every other row's scale differs); dense random blocks and blocks with
scales down to 2^-127 are within the GEMM tolerance."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close

pytestmark = pytest.mark.gpu


def _tile(nib, scales):
    """[B, 16, 128] codes and [B, 16, 4] scale bytes -> the tiled lane order
    (lane l = row l % 16 + 16 * chunk: the chunk's 32 codes as 16 bytes, the
    lower k in the low nibble, and that row's scale byte for the chunk)."""
    B = nib.shape[0]
    codes = O.pack_nibbles(nib).reshape(B, 16, 4, 16).transpose(0, 2, 1, 3).reshape(B, 1024)
    sc = np.ascontiguousarray(scales.transpose(0, 2, 1)).reshape(B, 64)
    return np.ascontiguousarray(codes), sc


def _run(na, sa, nb, sb):
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()
    ca, ea = _tile(na, sa)
    cb, eb = _tile(nb, sb)
    d = sq.check_mfma_fp4(dev(ca), dev(ea), dev(cb), dev(eb))
    torch.cuda.synchronize()
    return d.cpu().numpy()


def _ref(na, sa, nb, sb):
    a, b = O.dequant_mx(sa, na), O.dequant_mx(sb, nb)
    return a @ b.transpose(0, 2, 1), np.abs(a) @ np.abs(b).transpose(0, 2, 1)


def test_mfma_one_hot_lane_layout():
    print("mfma one-hot", flush=True)
    rng = np.random.default_rng(3)
    m0, n0, c = np.meshgrid(np.arange(16), np.arange(16), np.arange(4), indexing="ij")
    m0, n0, c = m0.ravel(), n0.ravel(), c.ravel()
    B = len(m0)
    k0 = c * 32 + (5 * m0 + 3 * n0) % 32                     # every position of every chunk
    assert len(np.unique(k0)) == 128
    nonzero = np.array([1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15], dtype=np.uint8)
    na = np.zeros((B, 16, 128), dtype=np.uint8)
    nb = np.zeros((B, 16, 128), dtype=np.uint8)
    na[np.arange(B), m0, k0] = rng.choice(nonzero, B)
    nb[np.arange(B), n0, k0] = rng.choice(nonzero, B)
    sa = rng.integers(100, 151, (B, 16, 4)).astype(np.uint8)  # every row's and chunk's scale different
    sb = rng.integers(100, 151, (B, 16, 4)).astype(np.uint8)
    d = _run(na, sa, nb, sb)
    ref, _ = _ref(na, sa, nb, sb)
    assert np.count_nonzero(ref) == B
    want = ref.astype(np.float32)                             # one product: exact in binary32
    bad = d != want
    assert not bad.any(), f"{int(bad.sum())} outputs differ; first block {np.argwhere(bad)[0]}"


def test_mfma_dense_random():
    print("mfma dense random", flush=True)
    rng = np.random.default_rng(4)
    B = 256
    na = rng.integers(0, 16, (B, 16, 128)).astype(np.uint8)
    nb = rng.integers(0, 16, (B, 16, 128)).astype(np.uint8)
    sa = rng.integers(118, 137, (B, 16, 4)).astype(np.uint8)
    sb = rng.integers(118, 137, (B, 16, 4)).astype(np.uint8)
    d = _run(na, sa, nb, sb)
    ref, bound = _ref(na, sa, nb, sb)
    assert_linear_close(d.reshape(-1, 16), ref.reshape(-1, 16), bound.reshape(-1, 16), "mfma dense")


def test_mfma_wide_scales_and_zero_operand():
    """Scales from 2^-127 (byte 0) to 2^13 on one operand, 2^-27 .. 2^0 on the
    other; and blocks whose second operand is all zero codes (+0 and -0) give
    exactly zero."""
    print("mfma wide scales", flush=True)
    rng = np.random.default_rng(5)
    B = 128
    na = rng.integers(0, 16, (B, 16, 128)).astype(np.uint8)
    nb = rng.integers(0, 16, (B, 16, 128)).astype(np.uint8)
    sa = rng.integers(0, 141, (B, 16, 4)).astype(np.uint8)
    sa[:, :, 0] = 0
    sb = rng.integers(100, 128, (B, 16, 4)).astype(np.uint8)
    nb[B // 2:] = rng.choice(np.array([0, 8], dtype=np.uint8), (B // 2, 16, 128))
    d = _run(na, sa, nb, sb)
    ref, bound = _ref(na, sa, nb, sb)
    assert_linear_close(d.reshape(-1, 16), ref.reshape(-1, 16), bound.reshape(-1, 16), "mfma wide scales")
    assert np.all(d[B // 2:] == 0.0)
