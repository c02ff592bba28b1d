/*
 * sharq.h -- C ABI of the SharQ linear-layer hot path for AMD Instinct MI355X (gfx950).
 *
 * The method (SharQ paper page, "SharQ: Bridging Activation Sparsity and FP4
 * Quantization for LLM Inference", Abstract): each activation row is split online
 * into an N:M-masked sparse backbone S, quantised to FP4, and a dense residual R
 * taken against the *quantised* backbone, also quantised to FP4.  A sparse FP4
 * GEMM on Q(S) and a dense FP4 GEMM on Q(R) read one shared FP4 weight payload,
 * and one epilogue sums them.  The preparation (normalisation, mask, residual,
 * both quantisations) is one fused operator.  The README page of the SharQ
 * repository (section "Evaluation") names the fused normalisation RMSNorm.
 *
 * Conventions for every entry point:
 *  - Ownership: the caller allocates every buffer (sizes from the *_bytes
 *    queries).  The library never allocates or frees device memory and holds
 *    no mutable global state other than a thread-local error string, a
 *    per-device architecture check, and the one device array per GPU that
 *    sharq_linear_grouped_noalloc uses as its workspace (see there), so every
 *    other entry point is reentrant.
 *  - Pointers named *_dev are device pointers; struct fields are device
 *    pointers unless stated.  `stream` is a hipStream_t (NULL = the null stream).
 *  - Ordering: every call is asynchronous on `stream`; nothing synchronises
 *    the host.
 *  - Errors: arguments are checked on the host before anything is launched; on
 *    any error nothing is launched and outputs are untouched.  No C++ exception
 *    crosses this ABI.  sharq_last_error() gives a thread-local detail string.
 *  - Inputs must be finite (NaN/Inf give unspecified codes).
 *  - FP4 codes are E2M1 nibbles, the lower k in the low nibble; the sign is
 *    nibble bit 3.  E8M0 scale bytes encode 2^(byte-127).
 *  - Tiled layout.  Every operand the GEMM reads is stored in blocks of 16
 *    rows x 128 K ("tiles"), in the lane order of the gfx950 block-scaled FP4
 *    MFMA: lane l of a tile is row 16*rb + l%16 and K range
 *    [128*kb + 32*(l/16), +32).  Rows are padded to RB*16 (RB = ceil(rows/16))
 *    and K to KB*128 (KB = ceil(K/128)); padding holds zero codes and zero
 *    scale bytes.  Per tile (rb, kb), tiles ordered rb-major then kb:
 *      codes          1024 B: lane l at 16*l (its 32 codes).  The backbone is
 *                             stored this way too, as a masked dense operand:
 *                             its kept codes in place, zero codes at the
 *                             dropped positions (gfx950 has no sparse FP4
 *                             MFMA; expanding a compressed form on chip cost
 *                             the GEMM more than the bytes it saves)
 *      2:4 metadata    256 B: lane l at 4*l, nibble g = group g of the lane
 *                             (the mask; the GEMM does not read it)
 *    Scale bytes are K-step-major: [KB][RB][64], byte l of (kb, rb) is the
 *    E8M0 of lane l's 32-block.  Canonical row-major arrays follow by
 *    un-tiling (the tests do exactly that before comparing).
 */
#ifndef SHARQ_H
#define SHARQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHARQ_ABI_VERSION 1

typedef enum {
  SHARQ_OK = 0,
  SHARQ_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad enum */
  SHARQ_ERR_UNSUPPORTED = 2, /* valid request the library does not run (e.g. HiF4, N:M != 2:4, not gfx950) */
  SHARQ_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  SHARQ_ERR_HIP = 4          /* a HIP runtime call or launch failed; detail in sharq_last_error() */
} sharq_status;

/* FP4 formats named by the SharQ abstract (it reports results in NVFP4, HiF4
 * and MXFP4).
 *  MXFP4 = OCP Microscaling v1.0: 32-element blocks, E8M0 scale.
 *  NVFP4 (the pages name it without a definition; this follows the public
 *  two-level NVFP4 description): E2M1 codes in 16-element blocks with an OCP
 *  E4M3 block scale (bias 7, subnormals, largest 448) and one binary32 scale
 *  per tensor.  For a tensor T (S, R or W, each separately) with largest
 *  magnitude A: g = A / 2688 (2688 = 6 * 448; g = 1 when A == 0); per block
 *  s = E4M3(amax_b / (6 g)) rounded to nearest even and saturated at 448;
 *  code = E2M1(u / (s g)), or the signed zero code when s == 0; value =
 *  val(code) * s * g.  Every step is one binary32 operation.  Tensors whose
 *  largest magnitude is nonzero but below 2^-126 are outside the supported
 *  range (their codes are unspecified).
 *  NVFP4 buffers: codes in the MX tiled layout; block scales tiled
 *  [KB][RB][128], lane l of a tile owning byte 2l (its first 16 elements) and
 *  2l+1 (the next 16); each scale buffer continues at the first 256-byte
 *  boundary after the block scales (offset round_up(KB*RB*128, 256)) with the
 *  binary32 tensor scale.  The residual's and the weight's scale buffers then
 *  hold scratch of the kernels that compute the scale (sizes from the
 *  *_bytes queries).
 *  HiF4 is not defined on the pages: every entry point returns
 *  SHARQ_ERR_UNSUPPORTED for it. */
typedef enum { SHARQ_FMT_MXFP4 = 0, SHARQ_FMT_NVFP4 = 1, SHARQ_FMT_HIF4 = 2 } sharq_format;

typedef enum { SHARQ_OUT_F32 = 0, SHARQ_OUT_BF16 = 1 } sharq_out_dtype;

/* Which GEMM path a weight scale view serves (SharQ paper page, Abstract:
 * both paths read one FP4 weight payload, each through its own scale view). */
typedef enum { SHARQ_PATH_SPARSE = 0, SHARQ_PATH_DENSE = 1 } sharq_path;

/* A scale view: how one GEMM path reads the weight's block scales.
 * base: device pointer to the tiled scale bytes (MXFP4: E8M0 [KB][NB][64];
 * NVFP4: E4M3 [KB][NB][128] followed by the tensor scale); ld: bytes between
 * K steps (NB*64 or NB*128); block: K elements per scale byte (32 or 16).
 * On gfx950 both paths run the same MFMA on dense 4-bit operands (the
 * backbone is a masked dense operand), so sharq_pack_weight sets both views
 * to the same array and layout. */
typedef struct {
  const uint8_t* base;
  int64_t ld;
  int32_t block;
  int32_t reserved;
} sharq_scale_view;

/* Packed weight W[N,K] (nn.Linear orientation: out x in; Y = X W^T).
 * The caller sets codes/scales to buffers of the queried sizes; sharq_pack_weight
 * fills them and every other field. */
typedef struct {
  uint32_t struct_size;     /* sizeof(sharq_weight) */
  uint32_t layout_version;  /* SHARQ_ABI_VERSION */
  int64_t N, K;
  int32_t fmt;              /* sharq_format */
  int32_t reserved;
  uint8_t* codes;           /* tiled dense codes, NB*KB tiles: the single FP4 payload both paths read */
  uint8_t* scales;          /* tiled E8M0 scales [KB][NB][64] */
  sharq_scale_view view[2]; /* indexed by sharq_path */
} sharq_weight;

/* Prepared activation (output of sharq_prepare), 2:4 and MXFP4, tiled layout:
 *   s_codes   codes of S: E2M1 of the kept entries in place, the zero code at
 *             dropped positions (RB*KB*1024 B)
 *   s_meta    2:4 metadata: per group of 4 the kept offsets i0<i1 as the
 *             nibble i0 | i1<<2 (RB*KB*256 B)
 *   s_scales  E8M0 of S per 32 logical positions ([KB][RB][64])
 *   r_codes   dense E2M1 of R (RB*KB*1024 B)
 *   r_scales  E8M0 of R ([KB][RB][64]) */
typedef struct {
  uint32_t struct_size;     /* sizeof(sharq_act) */
  uint32_t layout_version;  /* SHARQ_ABI_VERSION */
  int64_t M, K;
  int32_t n, m;             /* N:M pattern of the backbone mask */
  int32_t fmt;              /* sharq_format */
  int32_t reserved;
  uint8_t* s_codes;
  uint8_t* s_meta;
  uint8_t* s_scales;
  uint8_t* r_codes;
  uint8_t* r_scales;
} sharq_act;

/* ABI version of the loaded library (SHARQ_ABI_VERSION). */
int sharq_abi_version(void);

/* Text of a status code (static storage). */
const char* sharq_status_str(sharq_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* sharq_last_error(void);

/* Byte sizes of the packed weight buffers for W[N,K] in `fmt` (tiled:
 * codes NB*KB*1024; scales KB*NB*64 for MXFP4, for NVFP4 the E4M3 scales,
 * the tensor scale and scratch).
 * Errors: INVALID_ARG for N<=0, K<=0, K%32, null outputs; UNSUPPORTED for HiF4. */
sharq_status sharq_weight_bytes(int64_t N, int64_t K, int32_t fmt,
                                size_t* codes_bytes, size_t* scales_bytes);

/* Byte sizes of the five prepared-activation buffers, in the order
 * s_codes, s_meta, s_scales, r_codes, r_scales (MXFP4 tiled: RB*KB*{1024, 256,
 * 64, 1024, 64}; NVFP4: the scale buffers hold E4M3 scales, the tensor scale
 * and, for r_scales, the preparation's scratch).  M == 0 gives zeros.
 * Pattern (n,m) == (0,4) means no backbone: the plain FP4 linear (the dense
 * FP4 baseline SharQ is measured against); the three backbone sizes are 0.
 * Errors: INVALID_ARG for M<0, K<=0, K%32, null output; UNSUPPORTED unless
 * (n,m) == (2,4) with MXFP4 or NVFP4, or (n,m) == (0,4) with MXFP4. */
sharq_status sharq_act_bytes(int64_t M, int64_t K, int32_t n, int32_t m, int32_t fmt,
                             size_t sizes[5]);

/* Pack W[N,K] (bf16, row stride ldw elements) into the single FP4 weight
 * payload: MXFP4: per row n and 32-block b, E = floor(log2 amax)-2 (E8M0,
 * clamped) and E2M1 codes of w/2^E (round to nearest, ties to even,
 * saturating at 6); NVFP4: the tensor scale of all of W, then per row and
 * 16-block the E4M3 scale and codes (format rules above); written in the
 * tiled layout with zero padding.
 * SharQ abstract: both GEMM paths read this one payload.
 * `out` must have struct_size set and codes/scales pointing at buffers of the
 * sizes given by sharq_weight_bytes; N, K, fmt and both views are filled in.
 * Errors: INVALID_ARG (null, N<=0, K<=0, K%32, ldw<K, w not 16-B aligned or
 * ldw%8, a buffer not 16-B aligned), UNSUPPORTED (HiF4, device not gfx950),
 * HIP. */
sharq_status sharq_pack_weight(const void* w_bf16_dev, int64_t N, int64_t K, int64_t ldw,
                               int32_t fmt, sharq_weight* out, void* stream);

/* Fused preparation of X[M,K] (bf16, row stride ldx elements), one pass:
 *   v = RMSNorm(x) * gamma (binary32; skipped when gamma_bf16_dev is NULL):
 *       ss = pairwise tree sum of x^2 in index order over the row zero-padded
 *       to a power of two; inv = 1/sqrt(ss/K + eps), each op correctly rounded;
 *       v = (x*inv)*gamma;
 *   mask: in each group of 4 along K keep the 2 largest |v| (ties: lower index);
 *   S = v on kept entries, 0 elsewhere; Q(S) = MXFP4 over 32 logical positions;
 *   R = v - deq(Q(S)) (exact in binary32); Q(R) = MXFP4;
 *   all five outputs in the tiled layout, padding rows and K written as zeros.
 * With (n,m) == (0,4) there is no backbone: r_codes / r_scales receive the
 * MXFP4 of v itself and the s_* buffers are not used (they may be NULL).
 * With fmt == NVFP4 the quantiser is the NVFP4 one (blocks of 16 logical
 * positions; S's tensor scale from max|S|, R's from max|R|, so R's depends
 * on Q(S)); deq(Q(S)) = (val * s) * g in binary32.  This runs as three
 * dependent launches on `stream` (row statistics, backbone, residual).
 * SharQ paper page, Abstract: the normalisation, the mask and the residual
 * come out of one fused operator; the residual is taken against the
 * quantised backbone.
 * `out` must have struct_size set and the five buffers allocated per
 * sharq_act_bytes; M, K, n, m, fmt are filled in.  M == 0 launches nothing.
 * Errors: INVALID_ARG (null, K<=0, K%32, K>32768 with gamma, ldx<K, x not
 * 16-B aligned or ldx%8, gamma misaligned), UNSUPPORTED ((n,m) != (2,4),
 * HiF4, not gfx950), HIP. */
sharq_status sharq_prepare(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx,
                           const void* gamma_bf16_dev, float eps,
                           int32_t n, int32_t m, int32_t fmt,
                           sharq_act* out, void* stream);

/* Y[M,N] = deq(Q(S)) deq(W)^T + deq(Q(R)) deq(W)^T with one epilogue store.
 * SharQ abstract: a sparse FP4 GEMM on the backbone and a dense FP4 GEMM on
 * the residual; README "Benchmarks": the epilogue fusion sums them.
 * On gfx950 the backbone is a masked dense operand and both paths run
 * block-scaled MXFP4 MFMA into one fp32 accumulator, reading each weight tile
 * once for both paths.
 * An activation prepared with pattern 0:4 runs the dense GEMM alone:
 * Y = deq(Q(v)) deq(W)^T (the plain FP4 linear).
 * NVFP4: the E4M3 scales cannot ride the MX MFMA, so each code is expanded
 * on chip to val * s (exact in fp16), the fp16 MFMA accumulates each path in
 * fp32, and the epilogue applies the tensor scales:
 * y = g_S g_W acc_S + g_R g_W acc_R.  It is built for small M (decode); a
 * larger M reads the weight once per 64 rows.
 * y: device, fp32 or bf16 per out_dtype, row stride ldy elements (>= N).
 * Errors: INVALID_ARG (null, K mismatch, formats differ, scale views not those
 * of the format, ldy<N, misaligned y), UNSUPPORTED (HiF4, pattern, not
 * gfx950), HIP. */
sharq_status sharq_linear(const sharq_act* a, const sharq_weight* w,
                          void* y_dev, int64_t ldy, int32_t out_dtype, void* stream);

/* sharq_linear with the residual add of a decoder layer in its epilogue:
 * Y[m][n] = bf16(x[m][n] + y) for the layer's binary32 output y (one binary32
 * add, then round to nearest even) -- exactly sharq_linear (fp32 out) followed
 * by sharq_add_bf16_f32, without writing the fp32 output.
 * x: device bf16, row stride ldx >= N; Y: device bf16, row stride ldy >= N.
 * Y may be x itself (same pointer and stride; every element is read before it
 * is written by the same thread); any other overlap is undefined.  MXFP4
 * layers (2:4 or 0:4).
 * Errors: as sharq_linear, plus INVALID_ARG (null or misaligned x, ldx < N),
 * UNSUPPORTED (NVFP4-style). */
sharq_status sharq_linear_residual(const sharq_act* a, const sharq_weight* w, const void* x_bf16_dev, int64_t ldx,
                                   void* y_bf16_dev, int64_t ldy, void* stream);

/* Fusion ablations (README page of the SharQ repository, "Benchmarks": the
 * RMSNorm fusion and the epilogue fusion can each be switched off).
 *
 * sharq_rmsnorm: unfused RMSNorm of X[M,K] (bf16, row stride ldx) into
 * Y[M,K] (bf16, row stride ldy): the binary32 v of sharq_prepare (same
 * pairwise tree, same rounding steps) rounded to bf16 (nearest, ties to even).
 * Preparing Y with gamma NULL is the unfused preparation.
 * Errors: INVALID_ARG (null, M<0, K<=0, K%32, K>32768, ldx/ldy < K or not
 * multiples of 8 or > 2^26, buffers not 16-B aligned), UNSUPPORTED (not
 * gfx950), HIP. */
sharq_status sharq_rmsnorm(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx, const void* gamma_bf16_dev,
                           float eps, void* y_bf16_dev, int64_t ldy, void* stream);

/* out[i] = bf16(x[i] + y[i]) for n elements: x bf16, y fp32, the binary32 sum
 * rounded to nearest even (out may alias x): the residual add of the
 * synthetic decoder layer built from SharQ layers.
 * Errors: INVALID_ARG (null, n<0, misaligned), UNSUPPORTED (not gfx950), HIP. */
sharq_status sharq_add_bf16_f32(const void* x_bf16_dev, const float* y_dev, void* out_bf16_dev, int64_t n,
                                void* stream);

/* y[i] = a[i] + b[i] for n fp32 elements (device pointers; y may alias a or b):
 * the add of the unfused epilogue, whose two paths are two sharq_linear calls
 * on descriptors with pattern 0:4 whose r_codes / r_scales point at the
 * backbone's (s_codes / s_scales) or the residual's buffers.
 * Errors: INVALID_ARG (null, n<0, misaligned), UNSUPPORTED (not gfx950), HIP. */
sharq_status sharq_add_f32(const float* a_dev, const float* b_dev, float* y_dev, int64_t n, void* stream);

/* Gate/up projection of a gated MLP with the SwiGLU epilogue: the SharQ layer
 * Y = X W_gu^T on the packed [2F, K] weight whose 16-row blocks alternate gate
 * and up (block 2j = gate rows 16j..16j+15, block 2j+1 = up rows 16j..16j+15),
 * and one epilogue writes H[M,F] = bf16(SiLU(gate) * up) (binary32 SiLU
 * g / (1 + exp(-g)), then the product, rounded to nearest even) -- the bf16
 * input of the down projection's preparation, never materialising Y.
 * y: device bf16, row stride ldy >= F = N/2.  Runs the tiled kernel.
 * Errors: INVALID_ARG (null, shapes, N % 32, K mismatch, ldy, misaligned),
 * UNSUPPORTED (not 2:4 MXFP4, either operand's codes past 2 GiB -- the tiled
 * kernel's 31-bit offsets --, not gfx950), HIP. */
sharq_status sharq_linear_swiglu(const sharq_act* a, const sharq_weight* w, void* y_bf16_dev, int64_t ldy,
                                 void* stream);

/* The gate/up layer with the SwiGLU epilogue feeding the down projection's
 * preparation directly: *next = the prepared activation of H (2:4 mask,
 * MXFP4 of S and R, no RMSNorm) in the tiled layout, exactly what
 * sharq_linear_swiglu followed by sharq_prepare(H, gamma NULL) writes -- the
 * same bytes -- without storing H.  Each output tile of the GEMM stages its H
 * block in LDS and prepares whole 32-column blocks of it.
 * next: caller-owned buffers sized by sharq_act_bytes(M, N/2, 2, 4, MXFP4);
 * on success its M, K = N/2, n = 2, m = 4, fmt and layout_version are set.
 * Limits: 2:4 MXFP4, N/2 a multiple of 128 (others: UNSUPPORTED).
 * Errors: as sharq_linear_swiglu, plus INVALID_ARG (null next, next buffers
 * not set or not 16-byte aligned), UNSUPPORTED (N/2 % 128). */
sharq_status sharq_linear_swiglu_prep(const sharq_act* a, const sharq_weight* w, sharq_act* next, void* stream);

/* The whole layer in one launch for small M (decode): Y[M,N] of the bf16
 * activation X[M,K] (row stride ldx) and the packed weight, exactly
 * sharq_prepare followed by sharq_linear -- the same arithmetic, identical
 * outputs bit for bit -- without materialising the prepared activation: each
 * workgroup of the weight-streaming GEMM prepares the rows into LDS.  SharQ
 * abstract: the preparation is one fused operator feeding both GEMMs.
 * Limits: M <= 16, K <= 8192, 2:4, MXFP4 or NVFP4-style (others:
 * UNSUPPORTED; use the two-call path).  In the NVFP4-style format the
 * activation tensor is the M rows, so each workgroup also computes the two
 * tensor scales (g_S from max |v|, g_R from max |r|) itself, with the
 * preparation's arithmetic; the outputs equal sharq_prepare (fmt NVFP4)
 * followed by sharq_linear.  The MXFP4 form is faster than the two calls up to
 * M = 8 only.  gamma NULL skips RMSNorm.  y: fp32 or bf16 per out_dtype, row
 * stride ldy >= N.
 * Errors: INVALID_ARG (null, shapes, K mismatch, ldx/ldy, misaligned buffers,
 * weight views), UNSUPPORTED (limits, format, pattern, not gfx950), HIP. */
sharq_status sharq_linear_fused(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx,
                                const void* gamma_bf16_dev, float eps, int32_t n, int32_t m, int32_t fmt,
                                const sharq_weight* w, void* y_dev, int64_t ldy, int32_t out_dtype, void* stream);

/* Workspace bytes sharq_linear_grouped needs for `rows` routed rows, E
 * experts and reduction length K (the routed activation rows gathered into
 * expert order, each expert padded to whole 16-row blocks, plus small tables).
 * Errors: INVALID_ARG (null, rows<0, E<1 or E>1024, K<=0 or K%32). */
sharq_status sharq_grouped_workspace_bytes(int64_t rows, int32_t E, int64_t K, size_t* bytes);

/* Grouped expert layer (mixture of experts).  SharQ abstract: the method is
 * evaluated on mixture-of-experts models too; each expert is a SharQ linear
 * layer over the rows routed to it.
 *   a:          prepared activation of the source rows (e.g. the tokens, each
 *               prepared once: prep is row-local, so this equals preparing
 *               each routed copy);
 *   row_index:  device int32[rows]: routed row i reads source row
 *               row_index[i]; NULL means row i of `a` (then rows == a->M);
 *               an index outside [0, a->M) reads as an all-zero row;
 *   seg_offsets: device int64[E+1], nondecreasing, seg[0] = 0, seg[E] = rows:
 *               expert e owns routed rows [seg[e], seg[e+1]) (values outside
 *               that contract are clamped into it on the device);
 *   w:          the E experts' weights stacked along N and packed as one
 *               weight of N = E * N_e rows (sharq_pack_weight of the [E*N_e, K]
 *               stack); N_e must be a multiple of 16;
 *   y:          device [rows][ldy] (ldy >= N_e), row i = expert e's output for
 *               routed row i, in fp32 or bf16 per out_dtype;
 *   ws:         device workspace of ws_bytes >= sharq_grouped_workspace_bytes,
 *               owned by the caller; calls that share it must not overlap.
 * Errors: INVALID_ARG (null, shapes, K mismatch, ldy < N_e, workspace too
 * small, misaligned buffers), WORKSPACE, UNSUPPORTED (any format but MXFP4,
 * any pattern but 2:4, source or gathered activation codes or weight codes of
 * 2 GiB or more, not gfx950), HIP. */
sharq_status sharq_linear_grouped(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                  const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                  void* y_dev, int64_t ldy, int32_t out_dtype,
                                  void* ws_dev, size_t ws_bytes, void* stream);

/* The grouped gate/up layer of a mixture-of-experts MLP whose epilogue writes
 * the down projection's prepared activation (README page, section
 * "Benchmarks": epilogue fusion; the expert MLP as sharq_linear_swiglu_prep
 * computes it for a dense layer).  Arguments as sharq_linear_grouped, with
 * each expert's N_e = 2F weight rows interleaved in 16-row blocks (block 2j =
 * gate rows 16j..16j+15, block 2j+1 = the same up rows) and, instead of Y,
 *   next: output activation descriptor (struct_size set, all five buffers
 *         allocated per sharq_act_bytes(rows, F, 2, 4, MXFP4)); routed row i
 *         becomes row i of it: h = bf16(SiLU(gate) * up) of that row, then
 *         sharq_prepare(h, gamma = NULL), its padding rows as sharq_prepare
 *         writes them.  M, K = F, n, m, fmt are filled in.
 * The down projection then runs as sharq_linear_grouped(next, NULL, rows,
 * the same segment offsets, ...): its rows are already in expert order.
 * Errors: as sharq_linear_grouped; INVALID_ARG also for N_e % 32 or unset
 * output buffers; UNSUPPORTED for F % 128 (the K tiles of the next activation
 * hold no padding) or a format other than MXFP4. */
sharq_status sharq_linear_grouped_swiglu_prep(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                              const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                              sharq_act* next, void* ws_dev, size_t ws_bytes, void* stream);

/* sharq_linear_grouped for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, the same kernels and the same outputs, with the
 * workspace taken from a library-owned device array instead of an argument.
 * Each GPU the library runs on holds one such array of
 * sharq_noalloc_scratch_bytes() bytes (32 MiB) from the first use of the
 * library's code there until the process ends; the first call on a device
 * looks up its address once.  Nothing is allocated or freed per call.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from several host threads onto streams
 * that are not ordered) race and give undefined results.  Nothing in the array
 * needs to start at zero: every launch writes the parts it later reads.
 * Arguments as sharq_linear_grouped, without ws/ws_bytes.
 * Errors: as sharq_linear_grouped; WORKSPACE when the layer needs more than
 * the array holds (sharq_grouped_workspace_bytes(rows, E, K) >
 * sharq_noalloc_scratch_bytes()): use sharq_linear_grouped with a caller
 * workspace then. */
sharq_status sharq_linear_grouped_noalloc(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                          const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                          void* y_dev, int64_t ldy, int32_t out_dtype, void* stream);

/* Bytes of the library-owned scratch sharq_linear_grouped_noalloc uses on each GPU. */
size_t sharq_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H */
