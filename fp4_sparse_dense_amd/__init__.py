"""SharQ sparse-dense FP4 linear layer on AMD Instinct MI355X (gfx950).

Thin Python binding over libsharq.so (include/sharq.h).  Functions take torch
tensors only as device memory: every step of the layer runs in the HIP
kernels behind the C ABI.  The names follow the C entry points:

    w = sharq_pack_weight(w_bf16)                 # one FP4 weight payload
    a = sharq_prepare(x_bf16, gamma, eps)         # fused RMSNorm + 2:4 + MXFP4(S) + R + MXFP4(R)
    y = sharq_linear(a, w)                        # sparse + dense FP4 GEMMs, one epilogue
"""
from __future__ import annotations

import ctypes as C
import functools
import inspect

from . import _lib
from ._lib import FMT_HIF4, FMT_MXFP4, FMT_NVFP4, OUT_BF16, OUT_F32, SharqError

__all__ = [
    "SharqWeight", "SharqAct", "SharqError",
    "sharq_pack_weight", "sharq_prepare", "sharq_linear", "sharq_linear_grouped",
    "sharq_rmsnorm", "sharq_add_f32", "path_act", "grouped_workspace_bytes", "sharq_linear_fused",
    "sharq_linear_swiglu", "interleave_gate_up", "sharq_add_bf16_f32", "sharq_linear_residual",
    "sharq_linear_swiglu_prep", "peak_fp4_mfma", "peak_read",
    "sharq_linear_grouped_noalloc", "noalloc_scratch_bytes", "check_e2m1", "check_e4m3", "check_mfma_fp4", "sharq_linear_grouped_swiglu_prep",
    "weight_bytes", "act_bytes",
    "FMT_MXFP4", "FMT_NVFP4", "FMT_HIF4", "OUT_F32", "OUT_BF16",
]


def _torch():
    import torch
    return torch


def _on_stream(fn):
    """Run `fn` with torch's current stream set to its `stream` argument when
    one is given, so that every buffer it allocates (outputs, descriptors'
    buffers, the grouped workspace) belongs to the stream its kernels run on:
    the caching allocator then hands a freed block only to later work ordered
    on that stream, never to another stream while a kernel may still read it."""
    names = list(inspect.signature(fn).parameters)
    pos = names.index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        stream = kw.get("stream", args[pos] if len(args) > pos else None)
        if stream is None:
            return fn(*args, **kw)
        with _torch().cuda.stream(stream):
            return fn(*args, **kw)
    return wrapper


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def weight_bytes(N: int, K: int, fmt: int = FMT_MXFP4):
    lib = _lib.load()
    cb, sb = C.c_size_t(), C.c_size_t()
    _lib.check(lib.sharq_weight_bytes(N, K, fmt, C.byref(cb), C.byref(sb)), "sharq_weight_bytes")
    return cb.value, sb.value


def act_bytes(M: int, K: int, n: int = 2, m: int = 4, fmt: int = FMT_MXFP4):
    lib = _lib.load()
    sizes = (C.c_size_t * 5)()
    _lib.check(lib.sharq_act_bytes(M, K, n, m, fmt, sizes), "sharq_act_bytes")
    return list(sizes)


class SharqWeight:
    """Packed weight: flat device byte tensors `codes` and `scales` in the tiled
    layout of include/sharq.h, plus the descriptor."""

    def __init__(self, N: int, K: int, device, fmt: int = FMT_MXFP4):
        torch = _torch()
        cb, sb = weight_bytes(N, K, fmt)
        self.codes = torch.empty(cb, dtype=torch.uint8, device=device)
        self.scales = torch.empty(sb, dtype=torch.uint8, device=device)
        self.desc = _lib.WeightDesc()
        self.desc.struct_size = C.sizeof(_lib.WeightDesc)
        self.desc.codes = self.codes.data_ptr()
        self.desc.scales = self.scales.data_ptr()
        self.N, self.K, self.fmt = N, K, fmt


class SharqAct:
    """Prepared activation: five flat device byte tensors in the tiled layout of
    include/sharq.h, plus the descriptor."""

    FIELDS = ("s_codes", "s_meta", "s_scales", "r_codes", "r_scales")

    def __init__(self, M: int, K: int, device, n: int = 2, m: int = 4, fmt: int = FMT_MXFP4):
        torch = _torch()
        sizes = act_bytes(M, K, n, m, fmt)
        self.desc = _lib.ActDesc()
        self.desc.struct_size = C.sizeof(_lib.ActDesc)
        for name, size in zip(self.FIELDS, sizes):
            # keep every buffer 256-byte aligned even when empty
            t = torch.empty(max(size, 1), dtype=torch.uint8, device=device)[:size]
            setattr(self, name, t)
            setattr(self.desc, name, t.data_ptr())
        self.M, self.K, self.n, self.m, self.fmt = M, K, n, m, fmt

    def host(self) -> dict:
        """Copies of the five tiled byte arrays as numpy."""
        return {f: getattr(self, f).cpu().numpy() for f in self.FIELDS}


@_on_stream
def sharq_pack_weight(w, fmt: int = FMT_MXFP4, out: SharqWeight | None = None, stream=None) -> SharqWeight:
    """Pack a bf16 device weight [N, K] (row stride w.stride(0)) into the FP4 payload."""
    torch = _torch()
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D bf16 tensor with unit inner stride")
    N, K = w.shape
    out = out or SharqWeight(N, K, w.device, fmt)
    lib = _lib.load()
    _lib.check(lib.sharq_pack_weight(_ptr(w), N, K, w.stride(0), fmt, C.byref(out.desc), _stream_ptr(stream)),
               "sharq_pack_weight")
    return out


@_on_stream
def sharq_prepare(x, gamma=None, eps: float = 1e-5, n: int = 2, m: int = 4, fmt: int = FMT_MXFP4,
                  out: SharqAct | None = None, stream=None) -> SharqAct:
    """Fused preparation of bf16 device activations x [M, K]; gamma [K] bf16 or None (no RMSNorm)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit inner stride")
    if gamma is not None and (gamma.dtype != torch.bfloat16 or not gamma.is_contiguous()):
        raise ValueError("gamma must be a contiguous bf16 tensor")
    M, K = x.shape
    out = out or SharqAct(M, K, x.device, n, m, fmt)
    lib = _lib.load()
    _lib.check(lib.sharq_prepare(_ptr(x), M, K, x.stride(0), _ptr(gamma), eps, n, m, fmt, C.byref(out.desc),
                                 _stream_ptr(stream)), "sharq_prepare")
    return out


@_on_stream
def sharq_linear(act: SharqAct, weight: SharqWeight, out=None, out_dtype: int = OUT_F32, stream=None):
    """Y [M, N] = sparse FP4 GEMM + dense FP4 GEMM over the shared payload, one epilogue."""
    torch = _torch()
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(act.M, weight.N, dtype=dt, device=act.s_codes.device)
    if out.dtype != dt or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit inner stride and the requested dtype")
    lib = _lib.load()
    _lib.check(lib.sharq_linear(C.byref(act.desc), C.byref(weight.desc), _ptr(out), out.stride(0), out_dtype,
                                _stream_ptr(stream)), "sharq_linear")
    return out


@_on_stream
def sharq_linear_residual(act: SharqAct, weight: SharqWeight, x, out=None, stream=None):
    """Y [M, N] bf16 = bf16(x + layer output): the layer with the residual add
    in its epilogue (x: bf16 [M, N], unit inner stride; out may be x)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1 or tuple(x.shape) != (act.M, weight.N):
        raise ValueError("x must be a 2-D bf16 [M, N] tensor with unit inner stride")
    if out is None:
        out = torch.empty(act.M, weight.N, dtype=torch.bfloat16, device=act.r_codes.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be a 2-D bf16 tensor with unit inner stride")
    lib = _lib.load()
    _lib.check(lib.sharq_linear_residual(C.byref(act.desc), C.byref(weight.desc), _ptr(x), x.stride(0), _ptr(out),
                                         out.stride(0), _stream_ptr(stream)), "sharq_linear_residual")
    return out


def grouped_workspace_bytes(rows: int, experts: int, K: int) -> int:
    lib = _lib.load()
    n = C.c_size_t()
    _lib.check(lib.sharq_grouped_workspace_bytes(rows, experts, K, C.byref(n)), "sharq_grouped_workspace_bytes")
    return n.value


@_on_stream
def sharq_linear_grouped(act: SharqAct, weight: SharqWeight, seg_offsets, experts: int, row_index=None,
                         rows: int | None = None, out=None, out_dtype: int = OUT_F32, workspace=None, stream=None):
    """Grouped expert layer: expert e computes the SharQ linear layer of routed rows
    [seg[e], seg[e+1]) with its N_e = weight.N / experts rows of the stacked weight.

    seg_offsets: device int64 [E+1]; row_index: device int32 [rows] (routed row i
    reads activation row row_index[i]) or None (rows are the activation rows).
    Returns Y [rows, N_e]."""
    torch = _torch()
    dev = act.s_codes.device
    if rows is None:
        rows = int(row_index.numel()) if row_index is not None else act.M
    if seg_offsets.dtype != torch.int64 or not seg_offsets.is_contiguous() or seg_offsets.numel() != experts + 1:
        raise ValueError("seg_offsets must be a contiguous int64 tensor of E+1 entries")
    if row_index is not None and (row_index.dtype != torch.int32 or not row_index.is_contiguous()):
        raise ValueError("row_index must be a contiguous int32 tensor")
    ne = weight.N // experts
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(rows, ne, dtype=dt, device=dev)
    if out.dtype != dt or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit inner stride and the requested dtype")
    need = grouped_workspace_bytes(rows, experts, act.K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    lib = _lib.load()
    _lib.check(lib.sharq_linear_grouped(C.byref(act.desc), _ptr(row_index), rows, _ptr(seg_offsets), experts,
                                        C.byref(weight.desc), _ptr(out), out.stride(0), out_dtype,
                                        _ptr(workspace), workspace.numel(), _stream_ptr(stream)),
               "sharq_linear_grouped")
    return out


@_on_stream
def sharq_linear_grouped_noalloc(act: SharqAct, weight: SharqWeight, seg_offsets, experts: int, row_index=None,
                                 rows: int | None = None, out=None, out_dtype: int = OUT_F32, stream=None):
    """sharq_linear_grouped with the library's own per-GPU scratch as the
    workspace (include/sharq.h): the C entry point allocates nothing.  Pass
    `out` to allocate nothing here either.  Calls overlapping on one GPU race."""
    torch = _torch()
    dev = act.s_codes.device
    if rows is None:
        rows = int(row_index.numel()) if row_index is not None else act.M
    if seg_offsets.dtype != torch.int64 or not seg_offsets.is_contiguous() or seg_offsets.numel() != experts + 1:
        raise ValueError("seg_offsets must be a contiguous int64 tensor of E+1 entries")
    if row_index is not None and (row_index.dtype != torch.int32 or not row_index.is_contiguous()):
        raise ValueError("row_index must be a contiguous int32 tensor")
    ne = weight.N // experts
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(rows, ne, dtype=dt, device=dev)
    if out.dtype != dt or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit inner stride and the requested dtype")
    lib = _lib.load()
    _lib.check(lib.sharq_linear_grouped_noalloc(C.byref(act.desc), _ptr(row_index), rows, _ptr(seg_offsets), experts,
                                                C.byref(weight.desc), _ptr(out), out.stride(0), out_dtype,
                                                _stream_ptr(stream)), "sharq_linear_grouped_noalloc")
    return out


@_on_stream
def sharq_linear_grouped_swiglu_prep(act: SharqAct, weight: SharqWeight, seg_offsets, experts: int, row_index=None,
                                     rows: int | None = None, out: SharqAct | None = None, workspace=None,
                                     stream=None):
    """The grouped gate/up layer (each expert's gate and up rows interleaved as
    interleave_gate_up(..., experts=E) lays them out) whose epilogue prepares
    H = bf16(SiLU(gate) * up) for the down projection: returns the SharqAct of
    the routed rows in order, [rows, F] with F = N_e / 2, the same bytes as
    sharq_prepare of those rows of H.  Feed it to sharq_linear_grouped with
    row_index=None and the same seg_offsets."""
    torch = _torch()
    dev = act.s_codes.device
    if rows is None:
        rows = int(row_index.numel()) if row_index is not None else act.M
    if seg_offsets.dtype != torch.int64 or not seg_offsets.is_contiguous() or seg_offsets.numel() != experts + 1:
        raise ValueError("seg_offsets must be a contiguous int64 tensor of E+1 entries")
    if row_index is not None and (row_index.dtype != torch.int32 or not row_index.is_contiguous()):
        raise ValueError("row_index must be a contiguous int32 tensor")
    F = weight.N // experts // 2
    if out is None:
        out = SharqAct(rows, F, dev)
    if (out.M, out.K, out.n, out.m, out.fmt) != (rows, F, 2, 4, FMT_MXFP4):
        raise ValueError("out must be a 2:4 MXFP4 SharqAct of shape [rows, N_e/2]")
    need = grouped_workspace_bytes(rows, experts, act.K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    lib = _lib.load()
    _lib.check(lib.sharq_linear_grouped_swiglu_prep(C.byref(act.desc), _ptr(row_index), rows, _ptr(seg_offsets),
                                                    experts, C.byref(weight.desc), C.byref(out.desc),
                                                    _ptr(workspace), workspace.numel(), _stream_ptr(stream)),
               "sharq_linear_grouped_swiglu_prep")
    return out


def check_e2m1(x, exps, stream=None):
    """The kernels' E2M1 converts on device values (include/sharq_check.h):
    x float32 [S, n] (n % 8 == 0), exps int32 [S] (-127..125).  Returns
    (enc, pack, dec, unpack): uint32 [S, n/8] code words (value j of a group
    of eight in nibble j) of x / 2^e converted with the scale inside the
    convert and of the binary32 x * 2^-e converted with scale 1, and float32
    [S, n] values of those codes (times 2^e, and plain)."""
    torch = _torch()
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_contiguous() or x.shape[1] % 8:
        raise ValueError("x must be a contiguous float32 [S, n] tensor with n % 8 == 0")
    if exps.dtype != torch.int32 or not exps.is_contiguous() or exps.numel() != x.shape[0]:
        raise ValueError("exps must be a contiguous int32 tensor of S entries")
    S, n = x.shape
    enc = torch.empty(S, n // 8, dtype=torch.int32, device=x.device)
    pack = torch.empty_like(enc)
    dec = torch.empty_like(x)
    unpack = torch.empty_like(x)
    lib = _lib.load()
    _lib.check(lib.sharq_check_e2m1(_ptr(x), _ptr(exps), n, S, _ptr(enc), _ptr(pack), _ptr(dec), _ptr(unpack),
                                    _stream_ptr(stream)), "sharq_check_e2m1")
    return enc, pack, dec, unpack


def check_e4m3(x, stream=None):
    """The NVFP4-style kernels' E4M3 block-scale rounding (include/sharq_check.h)
    on a contiguous float32 device tensor of finite values >= 0.  Returns (byte
    uint8, value float32, decoded float32), each shaped like x."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_contiguous() or x.numel() < 1:
        raise ValueError("x must be a non-empty contiguous float32 tensor")
    byte = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    value = torch.empty_like(x)
    dec = torch.empty_like(x)
    lib = _lib.load()
    _lib.check(lib.sharq_check_e4m3(_ptr(x), x.numel(), _ptr(byte), _ptr(value), _ptr(dec), _stream_ptr(stream)),
               "sharq_check_e4m3")
    return byte, value, dec


def check_mfma_fp4(a, sa, b, sb, stream=None):
    """One FP4 MFMA per block as the GEMM kernels issue it (include/sharq_check.h):
    a, b uint8 [B, 1024] codes and sa, sb uint8 [B, 64] scale bytes in the tiled
    lane order.  Returns float32 [B, 16, 16], d[b][m][n]."""
    torch = _torch()
    for t, n in ((a, 1024), (b, 1024), (sa, 64), (sb, 64)):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.shape[1] != n or not t.is_contiguous():
            raise ValueError("a, b must be contiguous uint8 [B, 1024] and sa, sb uint8 [B, 64]")
    B = a.shape[0]
    if not (b.shape[0] == sa.shape[0] == sb.shape[0] == B):
        raise ValueError("operands hold different block counts")
    d = torch.empty(B, 16, 16, dtype=torch.float32, device=a.device)
    lib = _lib.load()
    _lib.check(lib.sharq_check_mfma_fp4(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), B, _ptr(d), _stream_ptr(stream)),
               "sharq_check_mfma_fp4")
    return d


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch sharq_linear_grouped_noalloc uses."""
    return int(_lib.load().sharq_noalloc_scratch_bytes())


@_on_stream
def sharq_rmsnorm(x, gamma, eps: float = 1e-5, out=None, stream=None):
    """Unfused RMSNorm (fusion ablation): bf16 [M, K] of the binary32 row the
    fused preparation computes, rounded to nearest even."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit inner stride")
    if gamma is None or gamma.dtype != torch.bfloat16 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bf16 tensor")
    M, K = x.shape
    if out is None:
        out = torch.empty(M, K, dtype=torch.bfloat16, device=x.device)
    lib = _lib.load()
    _lib.check(lib.sharq_rmsnorm(_ptr(x), M, K, x.stride(0), _ptr(gamma), eps, _ptr(out), out.stride(0),
                                 _stream_ptr(stream)), "sharq_rmsnorm")
    return out


@_on_stream
def sharq_add_f32(a, b, out=None, stream=None):
    """out = a + b for contiguous fp32 device tensors of one size (the unfused epilogue's add)."""
    torch = _torch()
    if a.dtype != torch.float32 or b.dtype != torch.float32 or a.numel() != b.numel():
        raise ValueError("a and b must be fp32 tensors of one size")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    if out is None:
        out = torch.empty_like(a)
    lib = _lib.load()
    _lib.check(lib.sharq_add_f32(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream_ptr(stream)), "sharq_add_f32")
    return out


class _PathAct:
    """One GEMM path of a prepared activation as a descriptor of pattern 0:4
    (the plain FP4 operand): the backbone's or the residual's codes and scales."""

    def __init__(self, act: SharqAct, path: str):
        codes, scales = (act.s_codes, act.s_scales) if path == "backbone" else (act.r_codes, act.r_scales)
        self.M, self.K, self.n, self.m, self.fmt = act.M, act.K, 0, 4, act.fmt
        self.s_codes = codes
        self._act = act
        self._desc = _lib.ActDesc()
        self._desc.struct_size = C.sizeof(_lib.ActDesc)
        self._desc.M, self._desc.K, self._desc.n, self._desc.m, self._desc.fmt = act.M, act.K, 0, 4, act.fmt
        self._desc.r_codes = codes.data_ptr()
        self._desc.r_scales = scales.data_ptr()

    @property
    def desc(self):
        # valid once the activation has been prepared by the library
        self._desc.layout_version = self._act.desc.layout_version
        return self._desc


def path_act(act: SharqAct, path: str):
    """Descriptor running one path of the dual GEMM alone (unfused epilogue):
    path is "backbone" or "residual"; pass it to sharq_linear."""
    if path not in ("backbone", "residual"):
        raise ValueError("path is 'backbone' or 'residual'")
    if act.n != 2 or act.fmt != FMT_MXFP4:
        raise ValueError("paths are split for 2:4 MXFP4 activations")
    return _PathAct(act, path)


@_on_stream
def sharq_linear_fused(x, weight: SharqWeight, gamma=None, eps: float = 1e-5, out=None, out_dtype: int = OUT_F32,
                       stream=None):
    """The whole layer in one launch for M <= 16 (decode): the result of
    sharq_prepare + sharq_linear, bit for bit, without the prepared activation.
    The format is the weight's (MXFP4 or NVFP4-style)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit inner stride")
    if gamma is not None and (gamma.dtype != torch.bfloat16 or not gamma.is_contiguous()):
        raise ValueError("gamma must be a contiguous bf16 tensor")
    M, K = x.shape
    dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(M, weight.N, dtype=dt, device=x.device)
    if out.dtype != dt or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be 2-D with unit inner stride and the requested dtype")
    lib = _lib.load()
    _lib.check(lib.sharq_linear_fused(_ptr(x), M, K, x.stride(0), _ptr(gamma), eps, 2, 4, weight.fmt,
                                      C.byref(weight.desc), _ptr(out), out.stride(0), out_dtype,
                                      _stream_ptr(stream)), "sharq_linear_fused")
    return out


def interleave_gate_up(w_gate, w_up, experts: int = 1):
    """[F, K] gate and up weights -> the [2F, K] stack sharq_linear_swiglu expects
    (16-row blocks alternating gate, up); pack it with sharq_pack_weight.  With
    experts=E the inputs are E experts' [F_e, K] weights stacked along rows
    ([E F_e, K] each) and every expert's rows are interleaved in place (the
    stack sharq_linear_grouped_swiglu_prep expects)."""
    torch = _torch()
    R, K = w_gate.shape
    if experts < 1 or R % experts or (R // experts) % 16 or tuple(w_up.shape) != (R, K):
        raise ValueError("gate and up must both be [E*F_e, K] with F_e % 16 == 0")
    F = R // experts
    g = w_gate.reshape(experts, F // 16, 16, K)
    u = w_up.reshape(experts, F // 16, 16, K)
    return torch.stack([g, u], dim=2).reshape(2 * R, K)


@_on_stream
def sharq_linear_swiglu(act: SharqAct, weight: SharqWeight, out=None, stream=None):
    """H [M, N/2] bf16 = SiLU(gate) * up of the interleaved gate/up SharQ layer."""
    torch = _torch()
    F = weight.N // 2
    if out is None:
        out = torch.empty(act.M, F, dtype=torch.bfloat16, device=act.r_codes.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be a 2-D bf16 tensor with unit inner stride")
    lib = _lib.load()
    _lib.check(lib.sharq_linear_swiglu(C.byref(act.desc), C.byref(weight.desc), _ptr(out), out.stride(0),
                                       _stream_ptr(stream)), "sharq_linear_swiglu")
    return out


@_on_stream
def sharq_linear_swiglu_prep(act: SharqAct, weight: SharqWeight, out: SharqAct | None = None, stream=None):
    """The gate/up layer whose SwiGLU epilogue prepares H = bf16(SiLU(gate) * up)
    for the down projection (2:4, MXFP4, no RMSNorm) without storing H: the
    same bytes as sharq_prepare(sharq_linear_swiglu(act, weight))."""
    F = weight.N // 2
    if out is None:
        out = SharqAct(act.M, F, act.r_codes.device)
    if (out.M, out.K, out.n, out.m, out.fmt) != (act.M, F, 2, 4, FMT_MXFP4):
        raise ValueError("out must be a 2:4 MXFP4 SharqAct of shape [M, N/2]")
    lib = _lib.load()
    _lib.check(lib.sharq_linear_swiglu_prep(C.byref(act.desc), C.byref(weight.desc), C.byref(out.desc),
                                            _stream_ptr(stream)), "sharq_linear_swiglu_prep")
    return out


def peak_fp4_mfma(operands, iters: int, sink, stream=None) -> float:
    """Launch the FP4 MFMA rate measurement (include/sharq_peak.h) on `stream`;
    returns the flops the launch executes.  operands: device uint8 tensor of
    >= 6144 bytes (0..4095 the first operands, 4096..6143 the second); sink:
    device float32 tensor of >= 1 element."""
    lib = _lib.load()
    flops = C.c_double()
    _lib.check(lib.sharq_peak_fp4_mfma(_ptr(operands), operands.numel(), iters, _ptr(sink), C.byref(flops),
                                       _stream_ptr(stream)), "sharq_peak_fp4_mfma")
    return flops.value


def peak_read(buf, sink, stream=None) -> float:
    """Launch the streaming read measurement over the device uint8 tensor `buf`
    (a multiple of 16 bytes, >= 1 MiB); returns the bytes the launch reads.
    sink: device int32 tensor of >= 1 element."""
    lib = _lib.load()
    nbytes = C.c_double()
    _lib.check(lib.sharq_peak_read(_ptr(buf), buf.numel(), _ptr(sink), C.byref(nbytes), _stream_ptr(stream)),
               "sharq_peak_read")
    return nbytes.value


@_on_stream
def sharq_add_bf16_f32(x, y, out=None, stream=None):
    """out = bf16(x + y): x bf16, y fp32 (contiguous, same size); the residual add."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or y.dtype != torch.float32 or x.numel() != y.numel():
        raise ValueError("x must be bf16 and y fp32, of one size")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise ValueError("x and y must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    lib = _lib.load()
    _lib.check(lib.sharq_add_bf16_f32(_ptr(x), _ptr(y), _ptr(out), x.numel(), _stream_ptr(stream)),
               "sharq_add_bf16_f32")
    return out
