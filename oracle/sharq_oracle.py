"""CPU oracle for the SharQ linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The HIP library never calls it and shares no code
with it; the two meet only through the seeded inputs of
``fp4_sparse_dense_amd.synth``.

What is computed (SharQ paper page, "SharQ: Bridging Activation Sparsity and
FP4 Quantization for LLM Inference", Abstract):

  per activation row: RMSNorm -> N:M mask keeping the largest magnitudes
  (the sparse backbone S) -> FP4 quantisation of S -> residual R = X - deq(Q(S))
  taken against the *quantised* backbone -> FP4 quantisation of R; then
  Y = deq(Q(S)) deq(W)^T + deq(Q(R)) deq(W)^T over one FP4 weight payload.

The pages print no formulas.  The readings this oracle takes of them:

* RMSNorm is evaluated in IEEE binary32 with the sum of squares taken as a
  balanced pairwise tree in index order over the row zero-padded to a power of
  two; 1/sqrt and the division by K are correctly rounded.
* Mask ties go to the lower index; +0 and -0 have equal magnitude.
* MXFP4 follows the OCP Microscaling v1.0 definition: 32-element blocks, E8M0
  shared exponent e = floor(log2 amax) - 2, E2M1 elements rounded to nearest
  with ties to the even code, saturating at 6.
* The residual is r = v - d in binary32 (exact: shown and tested).
* GEMM outputs are accumulated in float64.

Parity status of each function is given in its docstring ("pinned by" lists
the independent checks in tests/test_oracle_*.py).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# E2M1 magnitudes by 3-bit code (sign is bit 3 of the nibble).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
MX_BLOCK = 32
E8M0_BIAS = 127
E2M1_EMAX = 2          # largest E2M1 value is 1.5 * 2^2


# --------------------------------------------------------------------------
# bf16 widening
# --------------------------------------------------------------------------
def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the upper half of binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# RMSNorm  (SharQ abstract: the preparation operator absorbs the normalisation;
# SharQ README, Evaluation/Benchmarks: the fused normalisation is RMSNorm)
# --------------------------------------------------------------------------
def pairwise_tree_sum_f32(q: np.ndarray) -> np.ndarray:
    """Balanced pairwise sum along the last axis, binary32, in index order.

    The row is zero-padded to the next power of two P and summed as
    T[lo,hi) = T[lo,mid) + T[mid,hi), mid = (lo+hi)/2, leaves = elements.
    Pinned by: exact integer sums, fp64 comparison, explicit recursive tree.
    """
    q = np.asarray(q, dtype=F32)
    K = q.shape[-1]
    P = 1
    while P < K:
        P *= 2
    if P != K:
        pad = np.zeros(q.shape[:-1] + (P - K,), dtype=F32)
        q = np.concatenate([q, pad], axis=-1)
    while q.shape[-1] > 1:
        q = q[..., 0::2] + q[..., 1::2]
    return q[..., 0]


def rmsnorm(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """v = x * (1/sqrt(mean(x^2) + eps)) * gamma in binary32; gamma None -> v = x.

    Steps: x widened exactly; q = x*x (exact: 8-bit significands);
    ss = pairwise tree of q; mean = ss / K; inv = 1 / sqrt(mean + eps);
    v = (x * inv) * gamma, every operation rounded once to binary32.
    Pinned by: constant-row closed form, fp64 formula within 4 ulp,
    the identity path.
    """
    x = widen_bf16(x_bits)
    if gamma_bits is None:
        return x.copy()
    K = x.shape[-1]
    with np.errstate(over="ignore", divide="ignore"):    # IEEE overflow to inf is part of the definition
        ss = pairwise_tree_sum_f32(x * x)
        mean = ss / F32(K)
        inv = F32(1.0) / np.sqrt(mean + F32(eps))
    g = widen_bf16(gamma_bits)
    return (x * inv[..., None]) * g


# --------------------------------------------------------------------------
# N:M input-adaptive mask  (SharQ paper page, Abstract: a mask chosen per input
# keeps the largest-magnitude entries, the outliers, as the sparse backbone)
# --------------------------------------------------------------------------
def nm_mask(v: np.ndarray, n: int = 2, m: int = 4) -> np.ndarray:
    """Boolean keep-mask: in each aligned group of m along the last axis keep n.

    Element k of a group is kept iff fewer than n members beat it, where i
    beats k when |v_i| > |v_k|, or |v_i| == |v_k| and i < k.
    Pinned by: brute force over every 4-tuple of a 7-value set with ties and
    signed zeros; exactly-n and ordering invariants.
    """
    v = np.asarray(v, dtype=F32)
    K = v.shape[-1]
    if K % m:
        raise ValueError("K must be a multiple of m")
    a = np.abs(v).reshape(v.shape[:-1] + (K // m, m))
    rank = np.zeros(a.shape, dtype=np.int32)
    for k in range(m):
        for i in range(m):
            if i == k:
                continue
            beats = a[..., i] > a[..., k]
            if i < k:
                beats = beats | (a[..., i] == a[..., k])
            rank[..., k] += beats
    return (rank < n).reshape(v.shape)


def pack_meta_24(kept: np.ndarray) -> np.ndarray:
    """2:4 metadata: per group the two kept offsets i0 < i1 as nibble i0 | i1<<2;
    group j goes to byte j//2, low nibble for even j.  Shape [..., K/8] uint8."""
    K = kept.shape[-1]
    g = kept.reshape(kept.shape[:-1] + (K // 4, 4))
    if not np.all(g.sum(-1) == 2):
        raise ValueError("2:4 metadata needs exactly two kept per group")
    off = np.argsort(~g, axis=-1, kind="stable")[..., :2]   # kept offsets, ascending
    nib = (off[..., 0] | (off[..., 1] << 2)).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_meta_24(meta: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_meta_24: boolean keep-mask [..., K]."""
    meta = np.asarray(meta, dtype=np.uint8)
    nib = np.stack([meta & 0xF, meta >> 4], axis=-1).reshape(meta.shape[:-1] + (K // 4,))
    i0, i1 = nib & 3, nib >> 2
    pos = np.arange(4)
    kept = (pos == i0[..., None]) | (pos == i1[..., None])
    return kept.reshape(meta.shape[:-1] + (K,))


# --------------------------------------------------------------------------
# MXFP4 (OCP Microscaling v1.0: E2M1 elements, E8M0 scale per 32 elements)
# --------------------------------------------------------------------------
def floor_log2(a: np.ndarray) -> np.ndarray:
    """Exact floor(log2 a) for positive finite a (frexp: a = f 2^x, f in [0.5,1))."""
    _, x = np.frexp(np.asarray(a, dtype=np.float64))
    return x.astype(np.int32) - 1


def mx_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent e = clamp(floor(log2 amax) - 2, -127, 127); amax == 0 -> -127."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -E8M0_BIAS, dtype=np.int32)
    nz = amax > 0
    e[nz] = floor_log2(amax[nz]) - E2M1_EMAX
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS)


def e2m1_nearest(t) -> np.ndarray:
    """E2M1 nibble of real t: nearest grid magnitude, ties to the even code,
    magnitudes beyond 6 saturate to 6 (6 is the nearest grid point there);
    nibble = sign(t)<<3 | code, the sign taken from t's sign bit (-0 -> 0x8).

    Each midpoint between neighbouring grid values is a decision threshold:
    crossing it moves up one code; landing exactly on it moves up only when
    the upper code is even.  Comparisons are exact (t is binary32, compared in
    float64).  Pinned by: exact-rational argmin over the whole grid.
    """
    t = np.asarray(t, dtype=np.float64)
    a = np.abs(t)
    code = np.zeros(a.shape, dtype=np.uint8)
    for i in range(7):
        mid = 0.5 * (E2M1_GRID[i] + E2M1_GRID[i + 1])
        up_even = (i + 1) % 2 == 0
        code += (a > mid) | ((a == mid) & up_even)
    return code | (np.signbit(t).astype(np.uint8) << 3)


def e2m1_value(nib) -> np.ndarray:
    """Signed value of an E2M1 nibble (float64; -0.0 for 0x8)."""
    nib = np.asarray(nib, dtype=np.uint8)
    mag = E2M1_GRID[nib & 7]
    return np.where(nib & 8, -mag, mag)


def quantize_mx(u: np.ndarray):
    """MXFP4 quantisation along the last axis (length a multiple of 32).

    Returns (E8M0 scale bytes [..., K/32], nibbles [..., K]).  Element code =
    e2m1_nearest(u / 2^e) with e the block's shared exponent; the division is
    exact in float64.  Pinned by: amax/2^e in [4,8), codes on the grid,
    brute force of the element rounding, closed-form blocks.
    """
    u = np.asarray(u, dtype=F32)
    K = u.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = u.reshape(u.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    e = mx_exponent(amax)
    t = blocks / np.exp2(e.astype(np.float64))[..., None]
    nib = e2m1_nearest(t).reshape(u.shape)
    return (e + E8M0_BIAS).astype(np.uint8), nib


def dequant_mx(scales: np.ndarray, nib: np.ndarray) -> np.ndarray:
    """val(code) * 2^(E-127), float64, exact."""
    K = nib.shape[-1]
    e = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    val = e2m1_value(nib).reshape(nib.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return (val * np.exp2(e.astype(np.float64))[..., None]).reshape(nib.shape)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """Two codes per byte, the lower index in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    return np.stack([b & 0xF, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))


# --------------------------------------------------------------------------
# Preparation  (SharQ abstract: mask generation, residual construction and
# normalisation form one preparation operator)
# --------------------------------------------------------------------------
def prepare(x_bits, gamma_bits=None, eps: float = 1e-5, n: int = 2, m: int = 4):
    """Sparse-dense decomposition of activation rows (MXFP4, 2:4 outputs).

    Returns a dict with the canonical byte outputs
      s_codes  [M, K/4]  kept S codes in k order, 2 per byte (low nibble first)
      s_meta   [M, K/8]  2:4 metadata (pack_meta_24)
      s_scales [M, K/32] E8M0 of S over 32 logical positions
      r_codes  [M, K/2]  all R codes, 2 per byte
      r_scales [M, K/32] E8M0 of R
    and intermediates v, kept, s_nib (dense S nibbles), d (deq S, binary32),
    r (binary32).
    Pinned by: v == d + r exactly; S scale == scale of the unmasked block;
    exactly two kept per group; special cases that make R vanish.
    """
    if (n, m) != (2, 4):
        raise ValueError("byte outputs are defined for 2:4")
    v = rmsnorm(x_bits, gamma_bits, eps)
    kept = nm_mask(v, n, m)
    s = np.where(kept, v, F32(0.0))
    s_scales, s_nib = quantize_mx(s)
    d = dequant_mx(s_scales, s_nib)
    d = np.where(kept, d, 0.0).astype(F32)       # exact: at most 3 significant bits
    r = v - d                                      # binary32 subtraction
    r_scales, r_nib = quantize_mx(r)
    M, K = v.shape
    s_kept_nib = s_nib[kept].reshape(M, K // 2)
    return dict(
        s_codes=pack_nibbles(s_kept_nib),
        s_meta=pack_meta_24(kept),
        s_scales=s_scales,
        r_codes=pack_nibbles(r_nib),
        r_scales=r_scales,
        v=v, kept=kept, s_nib=s_nib, d=d, r=r,
    )


def pack_weight(w_bits):
    """Single FP4 weight payload (SharQ abstract: both paths read one FP4 weight
    payload): MXFP4 over each 32-block of a row of W[N,K] (bf16 bits), no mask,
    no norm.  Returns (codes [N, K/2], E8M0 scales [N, K/32])."""
    scales, nib = quantize_mx(widen_bf16(w_bits))
    return pack_nibbles(nib), scales


# --------------------------------------------------------------------------
# Dequantised operands and the dual GEMM
# --------------------------------------------------------------------------
def deq_sparse(s_codes, s_meta, s_scales, K: int) -> np.ndarray:
    """Dense float64 D^S [M,K] from the compressed 2:4 operand."""
    s_codes = np.asarray(s_codes)
    M = s_codes.shape[0]
    kept = unpack_meta_24(s_meta, K)
    nib = np.zeros((M, K), dtype=np.uint8)
    nib[kept] = unpack_nibbles(s_codes).reshape(-1)
    val = dequant_mx(s_scales, nib)
    return np.where(kept, val, 0.0)


def deq_dense(codes, scales) -> np.ndarray:
    return dequant_mx(scales, unpack_nibbles(codes))


def linear(act: dict, w_codes, w_scales, rows=None):
    """y = D^S D^W^T + D^R D^W^T in float64, plus the bound B = sum|terms|.

    (SharQ abstract: a sparse FP4 GEMM on the backbone and a dense FP4 GEMM on
    the residual; the README's epilogue fusion sums the two.)
    ``rows`` restricts the output to a subset of rows.  Returns (y, B).
    Pinned by: exact rational tiny GEMMs, the R == 0 special case,
    the path split y = y_S + y_R.
    """
    K = 2 * np.asarray(w_codes).shape[1]
    sl = slice(None) if rows is None else rows
    ds = deq_sparse(act["s_codes"][sl], act["s_meta"][sl], act["s_scales"][sl], K)
    dr = deq_dense(act["r_codes"][sl], act["r_scales"][sl])
    dw = deq_dense(w_codes, w_scales)
    y = ds @ dw.T + dr @ dw.T
    b = np.abs(ds) @ np.abs(dw).T + np.abs(dr) @ np.abs(dw).T
    return y, b


# --------------------------------------------------------------------------
# Fusion ablations (SharQ README, Benchmarks: the RMSNorm fusion and the
# epilogue fusion can be switched off).  Unfused RMSNorm writes the normalised
# row in bf16 and the preparation then runs without gamma; the unfused epilogue
# computes the two paths separately and adds them.
# --------------------------------------------------------------------------
def round_bf16(a) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest, ties to even (finite
    inputs): keep the upper 16 bits after adding 0x7FFF plus the kept LSB.
    Pinned by: exact rationals on neighbourhoods of midpoints, round trip."""
    u = np.asarray(a, dtype=F32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def rmsnorm_bf16(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """The unfused RMSNorm's output: bf16 bits of rmsnorm(x) (binary32)."""
    return round_bf16(rmsnorm(x_bits, gamma_bits, eps))


def residual_add_bf16(x_bits, y) -> np.ndarray:
    """The decoder layer's residual add: bf16 bits of (binary32 x + binary32 y)."""
    return round_bf16(widen_bf16(x_bits) + np.asarray(y, dtype=F32))


def linear_paths(act: dict, w_codes, w_scales, rows=None):
    """The two paths of the dual GEMM on their own (float64): (y_s, y_r, bound)."""
    K = 2 * np.asarray(w_codes).shape[1]
    sl = slice(None) if rows is None else rows
    ds = deq_sparse(act["s_codes"][sl], act["s_meta"][sl], act["s_scales"][sl], K)
    dr = deq_dense(act["r_codes"][sl], act["r_scales"][sl])
    dw = deq_dense(w_codes, w_scales)
    return ds @ dw.T, dr @ dw.T, np.abs(ds) @ np.abs(dw).T + np.abs(dr) @ np.abs(dw).T


# --------------------------------------------------------------------------
# Gate/up projection with the SwiGLU epilogue (a synthetic decoder layer's MLP
# front half; the SharQ README benchmarks whole decoder layers): the packed
# weight holds the gate and up rows in alternating 16-row blocks, and the
# layer's output is SiLU(gate) * up of the two SharQ outputs.
# --------------------------------------------------------------------------
def interleave_gate_up(w_gate, w_up) -> np.ndarray:
    """[2F, K] rows: block 2j = gate rows 16j..16j+15, block 2j+1 = the same up rows."""
    w_gate, w_up = np.asarray(w_gate), np.asarray(w_up)
    F, K = w_gate.shape
    if F % 16 or w_up.shape != (F, K):
        raise ValueError("gate and up must both be [F, K] with F % 16 == 0")
    return np.stack([w_gate.reshape(F // 16, 16, K), w_up.reshape(F // 16, 16, K)], axis=1).reshape(2 * F, K)


def silu(g) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def split_gate_up(y) -> tuple:
    """Columns of the interleaved layer output -> (gate [M, F], up [M, F])."""
    y = np.asarray(y)
    M, N2 = y.shape
    b = y.reshape(M, N2 // 32, 2, 16)
    return b[:, :, 0, :].reshape(M, N2 // 2), b[:, :, 1, :].reshape(M, N2 // 2)


def linear_swiglu(act: dict, w_codes, w_scales, rows=None):
    """SiLU(gate) * up (float64) of the interleaved gate/up SharQ layer, with the
    gate's and up's bounds sum|terms|.  Returns (h, b_gate, b_up, gate, up)."""
    y, b = linear(act, w_codes, w_scales, rows)
    g, u = split_gate_up(y)
    bg, bu = split_gate_up(b)
    return silu(g) * u, bg, bu, g, u


def swiglu_bound(g, u, bg, bu, rel: float = 1e-5, abs_: float = 1e-6) -> np.ndarray:
    """Allowed |h_gpu - h| for h = SiLU(g) u in bf16: the GEMM tolerance of g and u
    carried through (|SiLU'| <= 1.1), the binary32 evaluation (a few ulps), and
    the bf16 rounding (half an ulp: up to 2^-8 relative, for values just above a
    power of two -- bf16 carries 8 significant bits)."""
    eg, eu = rel * bg + abs_, rel * bu + abs_
    h = np.abs(silu(g) * u)
    return 1.1 * np.abs(u) * eg + np.abs(silu(g)) * eu + eg * eu + h * (2.0 ** -8 + 2.0 ** -20) + 1e-30


# --------------------------------------------------------------------------
# Plain FP4 linear: the comparator the SharQ README benchmarks against (its
# dense FP4 baseline mode): no backbone, the whole normalised row quantised
# once, one GEMM.  In the descriptors this is the N:M pattern 0:4.
# --------------------------------------------------------------------------
def prepare_dense(x_bits, gamma_bits=None, eps: float = 1e-5):
    """v = RMSNorm(x) (or x), then MXFP4 of v.  Returns r_codes [M, K/2] and
    r_scales [M, K/32] (the dense operand; the backbone arrays are empty) and v.
    Pinned by: per-element exact-rational codes and closed-form scales."""
    v = rmsnorm(x_bits, gamma_bits, eps)
    scales, nib = quantize_mx(v)
    return dict(r_codes=pack_nibbles(nib), r_scales=scales, v=v)


def linear_dense(act: dict, w_codes, w_scales, rows=None):
    """y = deq(Q(v)) deq(W)^T in float64 and the bound sum|terms|."""
    sl = slice(None) if rows is None else rows
    d = deq_dense(act["r_codes"][sl], act["r_scales"][sl])
    dw = deq_dense(w_codes, w_scales)
    return d @ dw.T, np.abs(d) @ np.abs(dw).T


# --------------------------------------------------------------------------
# NVFP4-style format: a reading.  The SharQ abstract reports the method under
# NVFP4 (and HiF4, MXFP4) but prints no definition; this follows the public
# two-level NVFP4 description: E2M1 elements in 16-element blocks, an OCP E4M3
# block scale, and one binary32 scale per tensor.
#   g_T = A_T / 2688 (A_T = max |u| over the whole tensor T; 2688 = 6 * 448,
#         the largest E2M1 times the largest E4M3), g_T = 1 when A_T = 0;
#   s_b = E4M3(amax_b / (6 g_T)), round to nearest even, saturating at 448;
#   code = E2M1(u / (s_b g_T)), or the signed zero code when s_b = 0;
#   value = val(code) * s_b * g_T.
# Every operation above is one binary32 operation, rounded once.  T is S, R
# and W separately, so the residual's tensor scale depends on Q(S).
# --------------------------------------------------------------------------
NV_BLOCK = 16
E4M3_MAX = 448.0
NV_TENSOR_DIV = F32(2688.0)


def e4m3_value(byte) -> np.ndarray:
    """Value of an OCP E4M3 byte with the sign bit clear (float64): exponent
    field E (bias 7) and mantissa m (3 bits); E = 0 is subnormal m * 2^-9;
    0x7F is NaN (excluded, never produced here)."""
    b = np.asarray(byte, dtype=np.int64) & 0x7F
    e = b >> 3
    m = (b & 7).astype(np.float64)
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))


def e4m3_round(x):
    """E4M3 of binary32 x >= 0: nearest representable value, ties to the even
    mantissa, values above 448 saturate to 448 (no infinity/NaN produced).

    Normal range (x >= 2^-6): the spacing is 2^(floor(log2 x) - 3); below it the
    spacing is the subnormal step 2^-9.  x / spacing is exact in float64 and
    np.rint rounds half to even.  Returns (value float64, byte uint8).
    Pinned by: brute force over all 127 non-negative E4M3 values on every
    midpoint and its binary32 neighbours, round trip of every byte.
    """
    x = np.asarray(x, dtype=F32).astype(np.float64)
    if np.any(x < 0) or not np.all(np.isfinite(x)):
        raise ValueError("e4m3_round takes finite x >= 0")
    step = np.full(x.shape, 2.0 ** -9)
    nrm = x >= 2.0 ** -6
    step[nrm] = np.exp2((floor_log2(x[nrm]) - 3).astype(np.float64))
    val = np.minimum(np.rint(x / step) * step, E4M3_MAX)
    byte = np.zeros(x.shape, dtype=np.uint8)
    nv = val >= 2.0 ** -6
    e = floor_log2(val[nv]) if np.any(nv) else np.zeros(0, np.int32)
    mant = (val[nv] / np.exp2(e.astype(np.float64)) - 1.0) * 8.0
    byte[nv] = ((e + 7) << 3).astype(np.uint8) | mant.astype(np.uint8)
    byte[~nv] = (val[~nv] / 2.0 ** -9).astype(np.uint8)
    return val, byte


def nv_tensor_scale(amax) -> np.float32:
    """g = A / 2688 in binary32; 1 for an all-zero tensor."""
    a = F32(amax)
    return F32(1.0) if a == 0 else F32(a / NV_TENSOR_DIV)


def quantize_nv(u: np.ndarray, g):
    """NVFP4-style quantisation along the last axis (length a multiple of 16)
    with tensor scale g.  Returns (E4M3 bytes [..., K/16], nibbles [..., K]).

    Per block: s = E4M3(amax / (6 * g)); t = s * g; code = E2M1(u / t)
    (binary32 quotient, then e2m1_nearest); s == 0 gives the signed zero code.
    Pinned by: closed-form block, the block-maximum-code invariant, exact
    rational brute force of each element's code.
    """
    u = np.asarray(u, dtype=F32)
    g = F32(g)
    K = u.shape[-1]
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    blocks = u.reshape(u.shape[:-1] + (K // NV_BLOCK, NV_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    sval, sbyte = e4m3_round(amax / (F32(6.0) * g))
    t = (sval.astype(F32) * g)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = blocks / t
    nib = e2m1_nearest(q)
    zero = np.broadcast_to((sbyte == 0)[..., None], blocks.shape)
    nib = np.where(zero, np.signbit(blocks).astype(np.uint8) << 3, nib)
    return sbyte, nib.reshape(u.shape)


def dequant_nv(scales: np.ndarray, nib: np.ndarray, g) -> np.ndarray:
    """val(code) * s * g in float64 (exact: at most 6 + 24 significant bits)."""
    K = nib.shape[-1]
    s = e4m3_value(scales)
    val = e2m1_value(nib).reshape(nib.shape[:-1] + (K // NV_BLOCK, NV_BLOCK))
    return (val * s[..., None] * np.float64(F32(g))).reshape(nib.shape)


def dequant_nv_f32(scales: np.ndarray, nib: np.ndarray, g) -> np.ndarray:
    """The binary32 dequantisation the residual uses: (val(code) * s) * g with
    val * s exact and one rounding for the product with g."""
    K = nib.shape[-1]
    s = e4m3_value(scales)
    vs = (e2m1_value(nib).reshape(nib.shape[:-1] + (K // NV_BLOCK, NV_BLOCK)) * s[..., None]).astype(F32)
    return (vs * F32(g)).reshape(nib.shape)


def prepare_nv(x_bits, gamma_bits=None, eps: float = 1e-5, n: int = 2, m: int = 4):
    """Sparse-dense decomposition in the NVFP4-style format (2:4 outputs).

    Same steps as prepare() with the quantiser replaced: S over 16 logical
    positions per block with tensor scale g_s = scale of max|S|; residual
    r = v - d in binary32 with d = (val * s) * g_s; R quantised with g_r =
    scale of max|r|.  Returns the byte outputs of prepare() (scales are E4M3
    per 16 positions, [M, K/16]) plus g_s, g_r and the intermediates.
    Pinned by: v == d + r exactly; max|S| == max|v|; the per-element code
    brute force of quantize_nv on both tensors; zero tensors.
    """
    if (n, m) != (2, 4):
        raise ValueError("byte outputs are defined for 2:4")
    v = rmsnorm(x_bits, gamma_bits, eps)
    kept = nm_mask(v, n, m)
    s = np.where(kept, v, F32(0.0))
    g_s = nv_tensor_scale(np.abs(s).max() if s.size else 0.0)
    s_scales, s_nib = quantize_nv(s, g_s)
    d = np.where(kept, dequant_nv_f32(s_scales, s_nib, g_s), F32(0.0)).astype(F32)
    r = v - d
    g_r = nv_tensor_scale(np.abs(r).max() if r.size else 0.0)
    r_scales, r_nib = quantize_nv(r, g_r)
    M, K = v.shape
    return dict(
        fmt="nvfp4",
        s_codes=pack_nibbles(s_nib[kept].reshape(M, K // 2)),
        s_meta=pack_meta_24(kept),
        s_scales=s_scales,
        r_codes=pack_nibbles(r_nib),
        r_scales=r_scales,
        g_s=g_s, g_r=g_r,
        v=v, kept=kept, s_nib=s_nib, d=d, r=r,
    )


def pack_weight_nv(w_bits):
    """NVFP4-style weight payload: g_w from max|W| over the whole tensor, then
    quantize_nv per row.  Returns (codes [N, K/2], E4M3 scales [N, K/16], g_w)."""
    u = widen_bf16(w_bits)
    g_w = nv_tensor_scale(np.abs(u).max())
    scales, nib = quantize_nv(u, g_w)
    return pack_nibbles(nib), scales, g_w


def linear_nv(act: dict, w_codes, w_scales, g_w, rows=None):
    """NVFP4-style dual GEMM: y = D^S D^W^T + D^R D^W^T with D = val * s * g
    (float64, exact), plus the bound B = sum|terms|.  Returns (y, B)."""
    K = 2 * np.asarray(w_codes).shape[1]
    sl = slice(None) if rows is None else rows
    kept = unpack_meta_24(act["s_meta"][sl], K)
    M = kept.shape[0]
    nib = np.zeros((M, K), dtype=np.uint8)
    nib[kept] = unpack_nibbles(act["s_codes"][sl]).reshape(-1)
    ds = np.where(kept, dequant_nv(act["s_scales"][sl], nib, act["g_s"]), 0.0)
    dr = dequant_nv(act["r_scales"][sl], unpack_nibbles(act["r_codes"][sl]), act["g_r"])
    dw = dequant_nv(w_scales, unpack_nibbles(w_codes), g_w)
    y = ds @ dw.T + dr @ dw.T
    b = np.abs(ds) @ np.abs(dw).T + np.abs(dr) @ np.abs(dw).T
    return y, b


def within_tolerance(y_gpu, y_ref, bound, rel: float = 1e-5, abs_: float = 1e-6):
    """Elementwise |y_gpu - y_ref| <= rel * sum|terms| + abs."""
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    lim = rel * bound + abs_
    return err <= lim
