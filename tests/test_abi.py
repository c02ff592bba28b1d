"""The C-ABI library loads, exports every function include/*.h declares,
answers size queries, and rejects invalid requests on the host before any HIP
call (CPU only: no compute call is made)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from fp4_sparse_dense_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(sharq_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsharq.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_match_header(lib):
    decl = declared_functions()
    assert "sharq_prepare" in decl and "sharq_linear" in decl and "sharq_pack_weight" in decl
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sharq_[a-z_0-9]+)", out))
    assert set(decl) <= exported, set(decl) - exported
    assert set(_lib.PROTOTYPES) == set(decl)
    for name in decl:
        getattr(lib, name)


def test_struct_sizes_match_c_layout():
    # sharq_scale_view: ptr + i64 + 2*i32 ; weight: 2*u32 + 2*i64 + 2*i32 + 2 ptr + 2 views
    assert C.sizeof(_lib.ScaleView) == 24
    assert C.sizeof(_lib.WeightDesc) == 8 + 16 + 8 + 16 + 48
    assert C.sizeof(_lib.ActDesc) == 8 + 16 + 8 + 8 + 40


def test_status_strings(lib):
    assert lib.sharq_abi_version() == _lib.SHARQ_ABI_VERSION
    assert lib.sharq_status_str(0) == b"ok"
    assert lib.sharq_status_str(2) == b"unsupported"


def test_size_queries(lib):
    cb, sb = C.c_size_t(), C.c_size_t()
    assert lib.sharq_weight_bytes(6144, 4096, 0, C.byref(cb), C.byref(sb)) == 0
    assert (cb.value, sb.value) == (6144 * 2048, 6144 * 128)
    sizes = (C.c_size_t * 5)()
    assert lib.sharq_act_bytes(2048, 4096, 2, 4, 0, sizes) == 0
    assert list(sizes) == [2048 * 2048, 2048 * 512, 2048 * 128, 2048 * 2048, 2048 * 128]
    # prep writes 1.1875 B per element: backbone and residual codes 0.5 each,
    # metadata 0.125, two scale bytes per 32
    assert sum(sizes) == int(2048 * 4096 * 1.1875)
    assert lib.sharq_act_bytes(0, 4096, 2, 4, 0, sizes) == 0 and sum(sizes) == 0


def test_size_queries_nvfp4(lib):
    """NVFP4-style: codes as MXFP4; block scales of two bytes per lane ([KB][RB][128])
    followed, at the next 256-byte boundary, by a 256-byte record holding the
    tensor scale; the residual's and the weight's records are followed by the
    kernels' scratch (per-row maxima and 1/rms, per-workgroup maxima)."""
    cb, sb = C.c_size_t(), C.c_size_t()
    assert lib.sharq_weight_bytes(4096, 4096, 1, C.byref(cb), C.byref(sb)) == 0
    NB, KB = 256, 32
    assert cb.value == 4096 * 2048
    assert sb.value == NB * KB * 128 + 256 + NB * (KB // 4) * 4
    sizes = (C.c_size_t * 5)()
    assert lib.sharq_act_bytes(8, 4096, 2, 4, 1, sizes) == 0
    RB = 1
    assert list(sizes)[0::2][:2] == [RB * KB * 1024, RB * KB * 128 + 256]
    assert sizes[1] == RB * KB * 256 and sizes[3] == RB * KB * 1024
    assert sizes[4] == RB * KB * 128 + 256 + 256 + 256 + 256
    assert lib.sharq_act_bytes(0, 4096, 2, 4, 1, sizes) == 0 and sum(sizes) == 0


def test_size_queries_plain_fp4(lib):
    """Pattern 0:4 (no backbone, the plain FP4 linear): only the dense operand."""
    sizes = (C.c_size_t * 5)()
    assert lib.sharq_act_bytes(2048, 4096, 0, 4, 0, sizes) == 0
    assert list(sizes) == [0, 0, 0, 2048 * 2048, 2048 * 128]
    assert lib.sharq_act_bytes(16, 4096, 0, 4, 1, sizes) == _lib.ERR_UNSUPPORTED   # MXFP4 only
    assert lib.sharq_act_bytes(16, 4096, 1, 4, 0, sizes) == _lib.ERR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    ((2048, 4008, 2, 4, 0), _lib.ERR_INVALID_ARG),   # K % 32
    ((2048, 0, 2, 4, 0), _lib.ERR_INVALID_ARG),
    ((-1, 4096, 2, 4, 0), _lib.ERR_INVALID_ARG),
    ((16, 4096, 1, 4, 0), _lib.ERR_UNSUPPORTED),     # only 2:4
    ((16, 4088, 2, 4, 1), _lib.ERR_INVALID_ARG),     # NVFP4 also needs K % 32
    ((16, 4096, 2, 4, 2), _lib.ERR_UNSUPPORTED),     # HiF4 undefined
    ((16, 4096, 2, 4, 7), _lib.ERR_INVALID_ARG),
])
def test_act_bytes_errors(lib, args, status):
    sizes = (C.c_size_t * 5)(*([123] * 5))
    assert lib.sharq_act_bytes(*args, sizes) == status
    assert list(sizes) == [123] * 5            # outputs untouched
    assert lib.sharq_last_error() != b""


def _act(M=16, K=256, **over):
    a = _lib.ActDesc()
    a.struct_size = C.sizeof(_lib.ActDesc)
    for i, f in enumerate(("s_codes", "s_meta", "s_scales", "r_codes", "r_scales")):
        setattr(a, f, 0x10000 * (i + 1))
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_prepare_rejects_before_launch(lib):
    x = C.c_void_p(0x100000)
    # bad struct size
    a = _act(struct_size=3)
    assert lib.sharq_prepare(x, 16, 256, 256, None, 1e-5, 2, 4, 0, C.byref(a), None) == _lib.ERR_INVALID_ARG
    a = _act()
    assert lib.sharq_prepare(x, 16, 250, 256, None, 1e-5, 2, 4, 0, C.byref(a), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_prepare(x, 16, 256, 200, None, 1e-5, 2, 4, 0, C.byref(a), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_prepare(C.c_void_p(0x100002), 16, 256, 256, None, 1e-5, 2, 4, 0, C.byref(a), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_prepare(x, 16, 256, 256, None, 1e-5, 3, 4, 0, C.byref(a), None) == _lib.ERR_UNSUPPORTED
    assert lib.sharq_prepare(x, 16, 256, 256, None, 1e-5, 2, 4, 2, C.byref(a), None) == _lib.ERR_UNSUPPORTED
    assert lib.sharq_prepare(x, 16, 65536, 65536, C.c_void_p(0x200000), 1e-5, 2, 4, 0, C.byref(a), None) == _lib.ERR_INVALID_ARG
    b = _act(s_meta=0)
    assert lib.sharq_prepare(x, 16, 256, 256, None, 1e-5, 2, 4, 0, C.byref(b), None) == _lib.ERR_INVALID_ARG
    assert b.M == 0 and b.layout_version == 0     # descriptor untouched on error
    # M == 0 is a valid no-op: no device is touched
    z = _act()
    assert lib.sharq_prepare(None, 0, 256, 256, None, 1e-5, 2, 4, 0, C.byref(z), None) == _lib.OK
    assert z.M == 0 and z.K == 256 and z.layout_version == _lib.SHARQ_ABI_VERSION


def test_pack_and_linear_reject_before_launch(lib):
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.codes, w.scales = 0x100000, 0x200000
    src = C.c_void_p(0x300000)
    assert lib.sharq_pack_weight(src, 16, 250, 256, 0, C.byref(w), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_pack_weight(src, 0, 256, 256, 0, C.byref(w), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_pack_weight(src, 16, 256, 100, 0, C.byref(w), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_pack_weight(src, 16, 256, 256, 2, C.byref(w), None) == _lib.ERR_UNSUPPORTED   # HiF4
    # linear: descriptors that were never filled by the library are refused
    a = _act()
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 16, 0, None) == _lib.ERR_INVALID_ARG
    a.layout_version = w.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m, w.N, w.K = 16, 256, 2, 4, 32, 512
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_INVALID_ARG
    w.K = 256
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 16, 0, None) == _lib.ERR_INVALID_ARG  # ldy < N
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 5, None) == _lib.ERR_INVALID_ARG
    # scale views must describe the MX payload
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_INVALID_ARG
    # well-formed views over two different scale arrays: refused as unsupported
    for p, base in ((0, 0x200000), (1, 0x210000)):
        w.view[p].base, w.view[p].ld, w.view[p].block = base, 2 * 64, 32
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_UNSUPPORTED
    # formats must agree; NVFP4-style descriptors need NVFP4-style views (block 16, stride NB*128)
    a.fmt, w.fmt = 1, 0
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_INVALID_ARG
    w.fmt = 1
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 2 * 64, 32
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_INVALID_ARG
    a.fmt = w.fmt = 2
    assert lib.sharq_linear(C.byref(a), C.byref(w), C.c_void_p(0x400000), 32, 0, None) == _lib.ERR_UNSUPPORTED
    a.fmt = w.fmt = 0
    a.M = 0
    assert lib.sharq_linear(C.byref(a), C.byref(w), None, 32, 0, None) == _lib.OK


def test_grouped_rejects_before_launch(lib):
    n = C.c_size_t()
    assert lib.sharq_grouped_workspace_bytes(100, 0, 256, C.byref(n)) == _lib.ERR_INVALID_ARG
    assert lib.sharq_grouped_workspace_bytes(100, 1025, 256, C.byref(n)) == _lib.ERR_INVALID_ARG
    assert lib.sharq_grouped_workspace_bytes(100, 8, 250, C.byref(n)) == _lib.ERR_INVALID_ARG
    assert lib.sharq_grouped_workspace_bytes(100, 8, 256, C.byref(n)) == _lib.OK
    # gathered rows of 8 experts padded to 16-row blocks: (100 + 8*15 + 15) // 16 blocks x 2 K tiles x 2176 B,
    # plus the segment tables and the block -> expert and tile -> expert maps (4 B per block and M tile)
    blocks, tiles = (100 + 8 * 15 + 15) // 16, (100 + 127) // 128 + 8
    assert n.value >= blocks * 2 * 2176 + 9 * (8 + 8 + 4) + 4 * (blocks + tiles)
    a = _act()
    a.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m = 64, 256, 2, 4
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.N, w.K, w.codes, w.scales = 8 * 16, 256, 0x100000, 0x200000   # 8 experts of 16 rows
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 8 * 64, 32
    seg, y, ws = C.c_void_p(0x500000), C.c_void_p(0x600000), C.c_void_p(0x700000)
    call = lambda rows, E, ri=None, ldy=32, wsb=1 << 30: lib.sharq_linear_grouped(
        C.byref(a), ri, rows, seg, E, C.byref(w), y, ldy, 0, ws, wsb, None)
    assert call(64, 0) == _lib.ERR_INVALID_ARG                   # E < 1
    assert call(64, 3) == _lib.ERR_INVALID_ARG                   # N is not 3 equal experts
    assert call(64, 16) == _lib.ERR_INVALID_ARG                  # N_e = 8, not a multiple of 16
    assert call(63, 8) == _lib.ERR_INVALID_ARG                   # rows != M without a row index
    assert call(64, 8, ldy=8) == _lib.ERR_INVALID_ARG            # ldy < N_e
    assert call(64, 8, wsb=100) == _lib.ERR_WORKSPACE            # workspace too small
    assert call(1 << 25, 8, ri=C.c_void_p(0x800000)) == _lib.ERR_UNSUPPORTED   # gathered codes past 2 GiB
    a.M = 1 << 25
    assert call(64, 8, ri=C.c_void_p(0x800000)) == _lib.ERR_UNSUPPORTED        # source codes past 2 GiB
    a.M = 64
    assert call(0, 8, ri=C.c_void_p(0x800000)) == _lib.OK        # nothing routed: no launch
    # the allocation-free form: the same checks, and a layer larger than the library's scratch
    na = lambda rows, E, ri=None, ldy=32: lib.sharq_linear_grouped_noalloc(
        C.byref(a), ri, rows, seg, E, C.byref(w), y, ldy, 0, None)
    assert lib.sharq_noalloc_scratch_bytes() == 32 << 20
    assert na(64, 3) == _lib.ERR_INVALID_ARG
    assert na(64, 8, ldy=8) == _lib.ERR_INVALID_ARG
    assert na(1 << 20, 8, ri=C.c_void_p(0x800000)) == _lib.ERR_WORKSPACE
    assert b"scratch" in lib.sharq_last_error()
    assert na(0, 8, ri=C.c_void_p(0x800000)) == _lib.OK           # nothing routed: no launch
    a.fmt = w.fmt = 1
    assert call(64, 8) == _lib.ERR_UNSUPPORTED                   # grouped layer is MXFP4 only
    a.fmt = w.fmt = 0
    a.n = 0
    assert call(64, 8) == _lib.ERR_UNSUPPORTED                   # and 2:4 only


def test_ablation_entry_points_reject_before_launch(lib):
    x, g, y = C.c_void_p(0x100000), C.c_void_p(0x200000), C.c_void_p(0x300000)
    assert lib.sharq_rmsnorm(x, 16, 250, 256, g, 1e-5, y, 256, None) == _lib.ERR_INVALID_ARG   # K % 32
    assert lib.sharq_rmsnorm(x, 16, 65536, 65536, g, 1e-5, y, 65536, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_rmsnorm(x, 16, 256, 256, None, 1e-5, y, 256, None) == _lib.ERR_INVALID_ARG  # gamma needed
    assert lib.sharq_rmsnorm(x, 16, 256, 256, g, 1e-5, y, 128, None) == _lib.ERR_INVALID_ARG     # ldy < K
    assert lib.sharq_rmsnorm(None, 0, 256, 256, None, 1e-5, None, 256, None) == _lib.OK          # M == 0
    assert lib.sharq_add_f32(x, g, y, -1, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_add_f32(None, g, y, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_add_f32(C.c_void_p(0x100002), g, y, 8, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_add_f32(None, None, None, 0, None) == _lib.OK


def test_fused_layer_rejects_before_launch(lib):
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.N, w.K, w.codes, w.scales = 64, 256, 0x100000, 0x200000
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 4 * 64, 32
    x, y = C.c_void_p(0x300000), C.c_void_p(0x400000)
    call = lambda M, K=256, n=2, fmt=0, ldy=64: lib.sharq_linear_fused(x, M, K, K, None, 1e-5, n, 4, fmt,
                                                                       C.byref(w), y, ldy, 0, None)
    assert call(17) == _lib.ERR_UNSUPPORTED                 # M <= 16
    assert call(4, n=0) == _lib.ERR_UNSUPPORTED             # 2:4 only
    assert call(4, fmt=1) == _lib.ERR_INVALID_ARG           # formats differ
    assert call(4, K=512) == _lib.ERR_INVALID_ARG           # K mismatch
    assert call(4, ldy=32) == _lib.ERR_INVALID_ARG          # ldy < N
    w.K = 16384
    assert call(4, K=16384) == _lib.ERR_UNSUPPORTED         # LDS limit
    assert call(0, K=16384) == _lib.ERR_UNSUPPORTED
    w.K = 256
    assert call(0) == _lib.OK                               # nothing to do


def test_swiglu_rejects_before_launch(lib):
    a = _act()
    a.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m = 64, 256, 2, 4
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.N, w.K, w.codes, w.scales = 48, 256, 0x100000, 0x200000
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 3 * 64, 32
    y = C.c_void_p(0x600000)
    assert lib.sharq_linear_swiglu(C.byref(a), C.byref(w), y, 24, None) == _lib.ERR_INVALID_ARG   # N % 32
    w.N = 64
    for p in (0, 1):
        w.view[p].ld = 4 * 64
    assert lib.sharq_linear_swiglu(C.byref(a), C.byref(w), y, 16, None) == _lib.ERR_INVALID_ARG   # ldy < N/2
    a.n = 0
    assert lib.sharq_linear_swiglu(C.byref(a), C.byref(w), y, 32, None) == _lib.ERR_UNSUPPORTED   # 2:4 only
    a.n, a.M = 2, 1 << 25
    assert lib.sharq_linear_swiglu(C.byref(a), C.byref(w), y, 32, None) == _lib.ERR_UNSUPPORTED   # codes past 2 GiB
    assert b"2 GiB" in lib.sharq_last_error()
    a.M = 0
    assert lib.sharq_linear_swiglu(C.byref(a), C.byref(w), y, 32, None) == _lib.OK


def test_residual_rejects_before_launch(lib):
    a = _act()
    a.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m = 64, 256, 2, 4
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.N, w.K, w.codes, w.scales = 64, 256, 0x100000, 0x200000
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 4 * 64, 32
    x, y = C.c_void_p(0x700000), C.c_void_p(0x600000)
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), None, 64, y, 64, None) == _lib.ERR_INVALID_ARG  # null x
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), x, 32, y, 64, None) == _lib.ERR_INVALID_ARG    # ldx < N
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), C.c_void_p(0x700001), 64, y, 64,
                                     None) == _lib.ERR_INVALID_ARG                                         # misaligned
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), x, 64, y, 32, None) == _lib.ERR_INVALID_ARG    # ldy < N
    a.fmt = w.fmt = 1
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), x, 64, y, 64, None) == _lib.ERR_UNSUPPORTED    # NVFP4-style
    a.fmt = w.fmt = 0
    a.M = 0
    assert lib.sharq_linear_residual(C.byref(a), C.byref(w), None, 64, None, 64, None) == _lib.OK


def test_swiglu_prep_rejects_before_launch(lib):
    a = _act()
    a.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m = 64, 256, 2, 4
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.N, w.K, w.codes, w.scales = 192, 256, 0x100000, 0x200000
    for p in (0, 1):
        w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, 12 * 64, 32
    nxt = _act()
    assert lib.sharq_linear_swiglu_prep(C.byref(a), C.byref(w), None, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_linear_swiglu_prep(C.byref(a), C.byref(w), C.byref(nxt), None) == _lib.ERR_UNSUPPORTED  # N/2 % 128
    w.N = 256
    for p in (0, 1):
        w.view[p].ld = 16 * 64
    nxt.r_codes = 0
    assert lib.sharq_linear_swiglu_prep(C.byref(a), C.byref(w), C.byref(nxt), None) == _lib.ERR_INVALID_ARG  # buffers
    a.M = 0
    assert lib.sharq_linear_swiglu_prep(C.byref(a), C.byref(w), C.byref(nxt), None) == _lib.OK
    assert (nxt.M, nxt.K, nxt.n, nxt.m) == (0, 128, 2, 4)


def test_grouped_swiglu_prep_rejects_before_launch(lib):
    a = _act()
    a.layout_version = _lib.SHARQ_ABI_VERSION
    a.M, a.K, a.n, a.m = 64, 256, 2, 4
    w = _lib.WeightDesc()
    w.struct_size = C.sizeof(_lib.WeightDesc)
    w.layout_version = _lib.SHARQ_ABI_VERSION
    w.K, w.codes, w.scales = 256, 0x100000, 0x200000

    def weight(n):
        w.N = n
        for p in (0, 1):
            w.view[p].base, w.view[p].ld, w.view[p].block = 0x200000, n // 16 * 64, 32

    seg, ws, ri = C.c_void_p(0x500000), C.c_void_p(0x700000), C.c_void_p(0x800000)
    nxt = _act()
    call = lambda rows, E, nx=nxt, wsb=1 << 30: lib.sharq_linear_grouped_swiglu_prep(
        C.byref(a), ri, rows, seg, E, C.byref(w), nx, ws, wsb, None)
    weight(2 * 256)                                              # 2 experts, N_e = 256, F = 128
    assert call(64, 2, nx=None) == _lib.ERR_INVALID_ARG          # no output descriptor
    assert call(64, 2, wsb=100) == _lib.ERR_WORKSPACE            # workspace too small
    weight(2 * 48)
    assert call(64, 2) == _lib.ERR_INVALID_ARG                   # N_e = 48: not pairs of 16-row blocks
    weight(2 * 64)
    assert call(64, 2) == _lib.ERR_UNSUPPORTED                   # F = 32: not a multiple of 128
    weight(2 * 256)
    bad = _act(r_codes=0)
    assert call(64, 2, nx=C.byref(bad)) == _lib.ERR_INVALID_ARG  # output buffers not set
    assert call(0, 2, nx=C.byref(nxt)) == _lib.OK                # nothing routed: no launch
    assert (nxt.M, nxt.K, nxt.n, nxt.m) == (0, 128, 2, 4)


def test_peak_entry_points_reject_bad_arguments(lib):
    """The measurement entry points check their arguments on the host."""
    d = C.c_double()
    buf = C.c_void_p(0x1000)
    assert lib.sharq_peak_fp4_mfma(None, 6144, 1, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_fp4_mfma(buf, 6128, 1, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_fp4_mfma(C.c_void_p(0x1004), 6144, 1, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_fp4_mfma(buf, 6144, 0, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_fp4_mfma(buf, 6144, (1 << 20) + 1, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert b"iters" in lib.sharq_last_error()
    assert lib.sharq_peak_read(buf, (1 << 20) - 16, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_read(buf, (1 << 20) + 8, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_peak_read(None, 1 << 20, buf, C.byref(d), None) == _lib.ERR_INVALID_ARG


def test_check_entry_points_reject_before_launch(lib):
    buf = C.c_void_p(0x100000)
    assert lib.sharq_check_e2m1(None, buf, 8, 1, buf, buf, buf, buf, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_check_e2m1(buf, buf, 12, 1, buf, buf, buf, buf, None) == _lib.ERR_INVALID_ARG   # n % 8
    assert lib.sharq_check_e2m1(buf, buf, 8, 0, buf, buf, buf, buf, None) == _lib.ERR_INVALID_ARG    # no scales
    assert lib.sharq_check_e4m3(None, 8, buf, buf, buf, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_check_e4m3(buf, 0, buf, buf, buf, None) == _lib.ERR_INVALID_ARG               # empty
    assert lib.sharq_check_e4m3(C.c_void_p(0x100002), 8, buf, buf, buf, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_check_mfma_fp4(None, buf, buf, buf, 1, buf, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_check_mfma_fp4(buf, buf, buf, buf, 0, buf, None) == _lib.ERR_INVALID_ARG        # no blocks
    assert lib.sharq_check_mfma_fp4(buf, buf, buf, buf, (1 << 20) + 1, buf, None) == _lib.ERR_INVALID_ARG
    assert lib.sharq_check_mfma_fp4(C.c_void_p(0x100008), buf, buf, buf, 1, buf, None) == _lib.ERR_INVALID_ARG
