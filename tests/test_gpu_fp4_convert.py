"""The hardware E2M1 converts behind every FP4 code the kernels write, checked
on the device against the rounding rule (SharQ paper page, Abstract: the
backbone and the residual are quantised to FP4; OCP MX v1.0 E2M1: round to
nearest, ties to the even code, saturating at 6, sign of zero kept).

Through sharq_check_e2m1 the GPU converts, exactly as the preparation (block
scale 2^e inside the convert), the weight pack and the NVFP4-style path
(binary32 product by 2^-e, then scale 1) use them:
  * every power-of-two block scale 2^e, e = -127 .. 125 (2^-127 is subnormal);
  * at each scale, every finite bf16 value, and the 64 binary32 neighbours on
    each side of every E2M1 grid point and decision midpoint times 2^e (both
    signs), plus 7 and 8 times 2^e (the top of a block's range).
The device only converts; the codes and values are compared here with the
oracle's e2m1_nearest / e2m1_value (exact in float64)."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from oracle import sharq_oracle as O

pytestmark = pytest.mark.gpu

POINTS = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0, 8.0])
EXPS = np.arange(-127, 126, dtype=np.int32)


def _bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    return (b << 16).view(np.float32)


def _neighbours(e):
    with np.errstate(over="ignore"):
        p = (POINTS * np.float64(2.0) ** int(e)).astype(np.float32)
    p = p[np.isfinite(p)]
    k = np.arange(-64, 65, dtype=np.int64)
    bits = p.view(np.uint32).astype(np.int64)[:, None] + k[None, :]
    bits = bits[(bits >= 0) & (bits < 0x7F800000)].astype(np.uint32)
    v = np.unique(bits).view(np.float32)
    return np.concatenate([v, -v])


def _nibbles(words):
    w = np.asarray(words).view(np.uint32)
    sh = (np.arange(8, dtype=np.uint32) * 4)
    return ((w[..., None] >> sh) & 0xF).astype(np.uint8).reshape(w.shape[0], -1)


def test_e2m1_converts_match_the_rounding_rule():
    import torch
    base = _bf16_finite()
    rows = [np.concatenate([base, _neighbours(e)]) for e in EXPS]
    n = max(len(r) for r in rows)
    n += (-n) % 8
    x = np.zeros((len(EXPS), n), dtype=np.float32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    print(f"e2m1 converts: {len(EXPS)} scales x {n} values", flush=True)
    xd = torch.from_numpy(x).cuda()
    enc, pack, dec, unpack = sq.check_e2m1(xd, torch.from_numpy(EXPS).cuda())
    torch.cuda.synchronize()
    enc_n, pack_n = _nibbles(enc.cpu().numpy()), _nibbles(pack.cpu().numpy())
    dec, unpack = dec.cpu().numpy(), unpack.cpu().numpy()
    scale = np.exp2(EXPS.astype(np.float64))[:, None]
    # the preparation: x / 2^e, exact in float64
    want = O.e2m1_nearest(x.astype(np.float64) / scale)
    bad = enc_n != want
    assert not bad.any(), f"{int(bad.sum())} codes differ, first at x={x[bad][0]!r} e={EXPS[np.nonzero(bad)[0][0]]}"
    want_dec = (O.e2m1_value(want) * scale).astype(np.float32)
    assert np.array_equal(dec.view(np.uint32), want_dec.view(np.uint32))
    # the pack and the NVFP4-style path: the binary32 product x * 2^-e (denormals kept; products past
    # the binary32 range are +-inf, which saturate to +-6 like any magnitude above 5), scale 1
    with np.errstate(over="ignore"):
        prod = x * (np.float64(1.0) / scale).astype(np.float32)
    want_p = O.e2m1_nearest(prod)
    bad = pack_n != want_p
    assert not bad.any(), f"{int(bad.sum())} pack codes differ, first at x={x[bad][0]!r}"
    assert np.array_equal(unpack.view(np.uint32), O.e2m1_value(want_p).astype(np.float32).view(np.uint32))
    # the sweep reaches every code at every scale where the grid fits binary32
    for i in (0, 127, len(EXPS) - 1):
        assert len(np.unique(enc_n[i])) == 16


def test_e4m3_rounding_matches_the_oracle():
    """The NVFP4-style kernels' E4M3 block-scale rounding and its decoding
    (through sharq_check_e4m3, which uses them as those kernels do) on every
    binary32 value in [2^-11, 480] -- where all of its rounding decisions lie,
    about 1.7e8 values -- and every 4096th pattern outside it up to the largest
    finite value, against the oracle's e4m3_round, value and byte."""
    import torch
    lo = int(np.float32(2.0 ** -11).view(np.uint32))
    hi = int(np.float32(480.0).view(np.uint32))
    print("e4m3 rounding: every binary32 in [2^-11, 480]", flush=True)
    for start, stop, step in ((0, lo, 4096), (hi, 0x7F800000, 4096), (lo, hi, 1)):
        for s0 in range(start, stop, step << 25):
            s1 = min(s0 + (step << 25), stop)
            x = torch.arange(s0, s1, step, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
            byte, value, dec = sq.check_e4m3(x)
            torch.cuda.synchronize()
            bits = np.arange(s0, s1, step, dtype=np.uint32)
            v, b = O.e4m3_round(bits.view(np.float32))
            gb = byte.cpu().numpy()
            bad = np.nonzero(gb != b)[0]
            assert bad.size == 0, f"x bits {int(bits[bad[0]]):#010x}: byte {int(gb[bad[0]]):#04x} != {int(b[bad[0]]):#04x}"
            assert np.array_equal(value.cpu().numpy().astype(np.float64), v)
            assert np.array_equal(dec.cpu().numpy().astype(np.float64), v)
