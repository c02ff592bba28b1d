"""Shared helpers for the GPU parity tests (device upload, comparison)."""
import numpy as np

from oracle import sharq_oracle as O

FIELDS = ("s_codes", "s_meta", "s_scales", "r_codes", "r_scales")


# ---------------------------------------------------------------------------
# Un-tiling: the GPU stores operands in blocks of 16 rows x 128 K in MFMA lane
# order (lane l = row l%16, 32-element chunk l/16); scales K-tile-major.  These
# numpy conversions recover the canonical row-major arrays of the oracle and
# check that all padding (rows past M, K past the end) holds what the method
# gives for zero input: zero codes and scales, metadata 0x44 (offsets 0, 1).
# ---------------------------------------------------------------------------
def _dims(rows, K):
    return -(-rows // 16), -(-K // 128)


def _crop(full, rows, cols, label, pad=0):
    assert np.all(full[rows:] == pad) and np.all(full[:, cols:] == pad), f"{label}: padding is not {pad:#x}"
    return full[:rows, :cols]


def untile_dense(buf, rows, K, label="codes"):
    RB, KB = _dims(rows, K)
    t = np.asarray(buf).reshape(RB, KB, 4, 16, 16).transpose(0, 3, 1, 2, 4)
    return _crop(t.reshape(RB * 16, KB * 64), rows, K // 2, label)


def untile_meta(buf, rows, K):
    RB, KB = _dims(rows, K)
    t = np.asarray(buf).reshape(RB, KB, 4, 16, 4).transpose(0, 3, 1, 2, 4)
    return _crop(t.reshape(RB * 16, KB * 16), rows, K // 8, "s_meta", pad=0x44)


def untile_scales(buf, rows, K, label="scales"):
    RB, KB = _dims(rows, K)
    t = np.asarray(buf).reshape(KB, RB, 4, 16).transpose(1, 3, 0, 2)
    return _crop(t.reshape(RB * 16, KB * 4), rows, K // 32, label)


def untile_act(raw: dict, M: int, K: int) -> dict:
    return dict(s_codes=untile_dense(raw["s_codes"], M, K, "s_codes"),
                s_meta=untile_meta(raw["s_meta"], M, K),
                s_scales=untile_scales(raw["s_scales"], M, K, "s_scales"),
                r_codes=untile_dense(raw["r_codes"], M, K, "r_codes"),
                r_scales=untile_scales(raw["r_scales"], M, K, "r_scales"))


def untile_weight(codes, scales, N, K):
    return untile_dense(codes, N, K, "w_codes"), untile_scales(scales, N, K, "w_scales")


def dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def assert_prep_equal(gpu: dict, ref: dict, label: str):
    """Byte-exact comparison of the five prepared arrays, with a readable first
    mismatch.  The GPU stores the backbone as a masked dense operand (kept codes
    in place, zero codes at dropped positions): that is the oracle's dense S
    nibbles, packed two per byte."""
    ref = dict(ref, s_codes=O.pack_nibbles(ref["s_nib"]))
    for f in FIELDS:
        g, r = gpu[f], ref[f]
        assert g.shape == r.shape, (label, f, g.shape, r.shape)
        bad = np.argwhere(g != r)
        if bad.size:
            i, j = bad[0]
            raise AssertionError(f"{label}: {f} differs at {len(bad)} bytes; first [{i},{j}] gpu={g[i, j]:#04x} "
                                 f"ref={r[i, j]:#04x}")


def assert_linear_close(y_gpu, y_ref, bound, label: str, extra=None):
    ok = O.within_tolerance(y_gpu, y_ref, bound) if extra is None else (
        np.abs(np.asarray(y_gpu, np.float64) - y_ref) <= 1e-5 * bound + 1e-6 + extra)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError(f"{label}: {int((~ok).sum())} outputs out of tolerance; first [{i},{j}] gpu={y_gpu[i, j]!r} "
                             f"ref={y_ref[i, j]!r} bound={bound[i, j]!r}")


# NVFP4-style buffers: two E4M3 bytes per lane ([KB][RB][64][2]), then at the
# next 256-byte boundary the binary32 tensor scale.
def untile_scales_nv(buf, rows, K, label="scales"):
    RB, KB = _dims(rows, K)
    raw = np.asarray(buf)
    t = raw[:KB * RB * 128].reshape(KB, RB, 4, 16, 2).transpose(1, 3, 0, 2, 4)
    scales = _crop(t.reshape(RB * 16, KB * 8), rows, K // 16, label)
    off = -(-KB * RB * 128 // 256) * 256
    g = raw[off:off + 4].copy().view(np.float32)[0]
    return scales, g


def untile_act_nv(raw: dict, M: int, K: int) -> dict:
    s_scales, g_s = untile_scales_nv(raw["s_scales"], M, K, "s_scales")
    r_scales, g_r = untile_scales_nv(raw["r_scales"], M, K, "r_scales")
    return dict(s_codes=untile_dense(raw["s_codes"], M, K, "s_codes"),
                s_meta=untile_meta(raw["s_meta"], M, K),
                s_scales=s_scales, r_codes=untile_dense(raw["r_codes"], M, K, "r_codes"),
                r_scales=r_scales, g_s=g_s, g_r=g_r)


def untile_weight_nv(codes, scales, N, K):
    s, g = untile_scales_nv(scales, N, K, "w_scales")
    return untile_dense(codes, N, K, "w_codes"), s, g
