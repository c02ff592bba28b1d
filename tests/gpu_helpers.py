"""Shared helpers for the GPU parity tests (device upload, comparison)."""
import numpy as np

from oracle import sharq_oracle as O

FIELDS = ("s_codes", "s_meta", "s_scales", "r_codes", "r_scales")


def dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def assert_prep_equal(gpu: dict, ref: dict, label: str):
    """Byte-exact comparison of the five prepared arrays, with a readable first mismatch."""
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
