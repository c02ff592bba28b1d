// C ABI of the SharQ hot path: argument checks, size queries, dispatch.
// Every check runs on the host before any HIP call, so invalid requests
// launch nothing and leave outputs untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sharq.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

sharq_status fail(sharq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

sharq_status hip_fail(hipError_t e, const char* what) {
  return fail(SHARQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// gfx950 check, once per device id (the only state the library keeps).
constexpr int kMaxDev = 64;
int g_arch_ok[kMaxDev];  // 0 unknown, 1 gfx950, -1 other
std::mutex g_arch_mu;

sharq_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(SHARQ_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    g_arch_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (g_arch_ok[dev] != 1) return fail(SHARQ_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return SHARQ_OK;
}

sharq_status check_fmt(int32_t fmt, bool nv_ok = true) {
  if (fmt == SHARQ_FMT_MXFP4) return SHARQ_OK;
  if (fmt == SHARQ_FMT_NVFP4)
    return nv_ok ? SHARQ_OK : fail(SHARQ_ERR_UNSUPPORTED, "the grouped expert layer is built for MXFP4 only");
  if (fmt == SHARQ_FMT_HIF4) return fail(SHARQ_ERR_UNSUPPORTED, "HiF4 is not defined on the SharQ pages");
  return fail(SHARQ_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
}

// Patterns built: 2:4, and 0:4 -- no backbone, the plain FP4 linear (MXFP4 only).
sharq_status check_pattern(int32_t n, int32_t m, int32_t fmt) {
  if (m == 4 && n == 2) return SHARQ_OK;
  if (m == 4 && n == 0)
    return fmt == SHARQ_FMT_MXFP4 ? SHARQ_OK
                                  : fail(SHARQ_ERR_UNSUPPORTED, "the plain FP4 linear (pattern 0:4) is built for MXFP4 only");
  return fail(SHARQ_ERR_UNSUPPORTED, "only the 2:4 pattern (and 0:4, no backbone) is built (got %d:%d)", (int)n, (int)m);
}

// the backbone buffers are needed (set and 16-byte aligned) unless the pattern is 0:4
bool backbone_ok(const sharq_act* a, int32_t n) {
  return n == 0 || (a->s_codes && a->s_meta && a->s_scales && aligned(a->s_codes, 16) &&
                    aligned(a->s_meta, 16) && aligned(a->s_scales, 16));
}

}  // namespace

namespace sharq {
// the thread-local detail string of sharq_last_error, for the other entry-point files
sharq_status record_error(sharq_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace sharq

extern "C" {

int sharq_abi_version(void) { return SHARQ_ABI_VERSION; }

const char* sharq_status_str(sharq_status s) {
  switch (s) {
    case SHARQ_OK: return "ok";
    case SHARQ_ERR_INVALID_ARG: return "invalid argument";
    case SHARQ_ERR_UNSUPPORTED: return "unsupported";
    case SHARQ_ERR_WORKSPACE: return "workspace too small";
    case SHARQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* sharq_last_error(void) { return g_err; }

sharq_status sharq_weight_bytes(int64_t N, int64_t K, int32_t fmt, size_t* codes_bytes,
                                size_t* scales_bytes) {
  g_err[0] = 0;
  if (!codes_bytes || !scales_bytes) return fail(SHARQ_ERR_INVALID_ARG, "null output pointer");
  if (N <= 0 || K <= 0) return fail(SHARQ_ERR_INVALID_ARG, "N and K must be positive (N=%lld K=%lld)", (long long)N, (long long)K);
  if (K % 32) return fail(SHARQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 32", (long long)K);
  sharq_status s = check_fmt(fmt);
  if (s) return s;
  const size_t nb = (size_t)((N + 15) / 16), kb = (size_t)((K + 127) / 128);
  *codes_bytes = nb * kb * 1024;
  *scales_bytes = fmt == SHARQ_FMT_NVFP4 ? sharq::nv_weight_layout(N, K).bytes : nb * kb * 64;
  return SHARQ_OK;
}

sharq_status sharq_act_bytes(int64_t M, int64_t K, int32_t n, int32_t m, int32_t fmt, size_t sizes[5]) {
  g_err[0] = 0;
  if (!sizes) return fail(SHARQ_ERR_INVALID_ARG, "null output pointer");
  if (M < 0 || K <= 0) return fail(SHARQ_ERR_INVALID_ARG, "bad shape M=%lld K=%lld", (long long)M, (long long)K);
  if (K % 32) return fail(SHARQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 32", (long long)K);
  sharq_status s = check_fmt(fmt);
  if (s) return s;
  s = check_pattern(n, m, fmt);
  if (s) return s;
  const size_t tiles = (size_t)((M + 15) / 16) * (size_t)((K + 127) / 128);
  sizes[0] = tiles * 1024;
  sizes[1] = tiles * 256;
  sizes[2] = tiles * 64;
  sizes[3] = tiles * 1024;
  sizes[4] = tiles * 64;
  if (fmt == SHARQ_FMT_NVFP4) {
    const sharq::NvActLayout L = sharq::nv_act_layout(M, K);
    sizes[2] = M > 0 ? L.s_bytes : 0;
    sizes[4] = M > 0 ? L.r_bytes : 0;
  }
  if (n == 0) sizes[0] = sizes[1] = sizes[2] = 0;   // no backbone
  return SHARQ_OK;
}

sharq_status sharq_pack_weight(const void* w_bf16_dev, int64_t N, int64_t K, int64_t ldw, int32_t fmt,
                               sharq_weight* out, void* stream) {
  g_err[0] = 0;
  if (!w_bf16_dev || !out) return fail(SHARQ_ERR_INVALID_ARG, "null pointer");
  if (out->struct_size != sizeof(sharq_weight))
    return fail(SHARQ_ERR_INVALID_ARG, "sharq_weight.struct_size %u != %zu", out->struct_size, sizeof(sharq_weight));
  if (!out->codes || !out->scales) return fail(SHARQ_ERR_INVALID_ARG, "weight buffers not set");
  if (N <= 0 || K <= 0 || K % 32) return fail(SHARQ_ERR_INVALID_ARG, "bad shape N=%lld K=%lld (K%%32 must be 0)", (long long)N, (long long)K);
  if (K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "K too large");
  if (ldw < K || ldw % 8) return fail(SHARQ_ERR_INVALID_ARG, "ldw=%lld must be >= K and a multiple of 8", (long long)ldw);
  if (!aligned(w_bf16_dev, 16)) return fail(SHARQ_ERR_INVALID_ARG, "weight not 16-byte aligned");
  if (!aligned(out->codes, 16) || !aligned(out->scales, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "weight buffers must be 16-byte aligned");
  sharq_status s = check_fmt(fmt);
  if (s) return s;
  s = check_device();
  if (s) return s;
  const bool nv = fmt == SHARQ_FMT_NVFP4;
  hipError_t e = nv ? sharq::launch_pack_weight_nv(static_cast<const uint16_t*>(w_bf16_dev), N, (int)K, ldw,
                                                   out->codes, out->scales, static_cast<hipStream_t>(stream))
                    : sharq::launch_pack_weight(static_cast<const uint16_t*>(w_bf16_dev), N, (int)K, ldw,
                                                out->codes, out->scales, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack_weight launch");
  out->layout_version = SHARQ_ABI_VERSION;
  out->N = N;
  out->K = K;
  out->fmt = fmt;
  for (int p = 0; p < 2; ++p) {
    out->view[p].base = out->scales;
    out->view[p].ld = (N + 15) / 16 * (nv ? 128 : 64);   // bytes between K tiles of the tiled scale array
    out->view[p].block = nv ? 16 : 32;
    out->view[p].reserved = 0;
  }
  return SHARQ_OK;
}

sharq_status sharq_prepare(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx, const void* gamma_bf16_dev,
                           float eps, int32_t n, int32_t m, int32_t fmt, sharq_act* out, void* stream) {
  g_err[0] = 0;
  if (!out) return fail(SHARQ_ERR_INVALID_ARG, "null output descriptor");
  if (out->struct_size != sizeof(sharq_act))
    return fail(SHARQ_ERR_INVALID_ARG, "sharq_act.struct_size %u != %zu", out->struct_size, sizeof(sharq_act));
  if (M < 0 || K <= 0 || K % 32) return fail(SHARQ_ERR_INVALID_ARG, "bad shape M=%lld K=%lld (K%%32 must be 0)", (long long)M, (long long)K);
  if (K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "K too large");
  if (gamma_bf16_dev && K > 32768) return fail(SHARQ_ERR_INVALID_ARG, "RMSNorm rows are limited to K <= 32768");
  if (ldx > (int64_t(1) << 26)) return fail(SHARQ_ERR_INVALID_ARG, "ldx=%lld exceeds 2^26 elements", (long long)ldx);
  sharq_status s = check_fmt(fmt);
  if (s) return s;
  s = check_pattern(n, m, fmt);
  if (s) return s;
  if (M > 0) {
    if (!x_bf16_dev) return fail(SHARQ_ERR_INVALID_ARG, "null activation pointer");
    if (!out->r_codes || !out->r_scales || !backbone_ok(out, n))
      return fail(SHARQ_ERR_INVALID_ARG, "activation output buffers not set or not 16-byte aligned");
    if (ldx < K || ldx % 8) return fail(SHARQ_ERR_INVALID_ARG, "ldx=%lld must be >= K and a multiple of 8", (long long)ldx);
    if (!aligned(x_bf16_dev, 16)) return fail(SHARQ_ERR_INVALID_ARG, "activation not 16-byte aligned");
    if (gamma_bf16_dev && !aligned(gamma_bf16_dev, 16)) return fail(SHARQ_ERR_INVALID_ARG, "gamma not 16-byte aligned");
    if (!aligned(out->r_codes, 16) || !aligned(out->r_scales, 16))
      return fail(SHARQ_ERR_INVALID_ARG, "activation output buffers must be 16-byte aligned");
    s = check_device();
    if (s) return s;
    sharq::PrepOut po{out->s_codes, out->s_meta, out->s_scales, out->r_codes, out->r_scales};
    hipError_t e = n == 0 ? sharq::launch_prepare_dense(static_cast<const uint16_t*>(x_bf16_dev), M, (int)K, ldx,
                                                        static_cast<const uint16_t*>(gamma_bf16_dev), eps, po,
                                                        static_cast<hipStream_t>(stream))
                   : fmt == SHARQ_FMT_NVFP4
                       ? sharq::launch_prepare_nv(static_cast<const uint16_t*>(x_bf16_dev), M, (int)K, ldx,
                                                  static_cast<const uint16_t*>(gamma_bf16_dev), eps, po,
                                                  static_cast<hipStream_t>(stream))
                       : sharq::launch_prepare(static_cast<const uint16_t*>(x_bf16_dev), M, (int)K, ldx,
                                               static_cast<const uint16_t*>(gamma_bf16_dev), eps, po,
                                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prepare launch");
  }
  out->layout_version = SHARQ_ABI_VERSION;
  out->M = M;
  out->K = K;
  out->n = n;
  out->m = m;
  out->fmt = fmt;
  return SHARQ_OK;
}

// sharq_linear and sharq_linear_residual: resid == nullptr for the plain layer
static sharq_status linear_impl(const sharq_act* a, const sharq_weight* w, void* y_dev, int64_t ldy, int32_t out_dtype,
                                const void* resid, int64_t ld_resid, void* stream) {
  if (!a || !w) return fail(SHARQ_ERR_INVALID_ARG, "null descriptor");
  if (a->struct_size != sizeof(sharq_act) || w->struct_size != sizeof(sharq_weight))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor struct_size mismatch");
  if (a->layout_version != SHARQ_ABI_VERSION || w->layout_version != SHARQ_ABI_VERSION)
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor layout_version mismatch (not produced by this library?)");
  if (a->K != w->K) return fail(SHARQ_ERR_INVALID_ARG, "K mismatch: activation %lld, weight %lld", (long long)a->K, (long long)w->K);
  if (a->M < 0 || w->N <= 0 || a->K <= 0 || a->K % 32) return fail(SHARQ_ERR_INVALID_ARG, "bad shapes");
  if (a->K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "K too large");
  if (out_dtype != SHARQ_OUT_F32 && out_dtype != SHARQ_OUT_BF16) return fail(SHARQ_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dtype);
  if (a->fmt != w->fmt) return fail(SHARQ_ERR_INVALID_ARG, "activation and weight formats differ");
  sharq_status s = check_fmt(a->fmt);
  if (s) return s;
  s = check_pattern(a->n, a->m, a->fmt);
  if (s) return s;
  if (a->M == 0) return SHARQ_OK;
  if (!y_dev) return fail(SHARQ_ERR_INVALID_ARG, "null output pointer");
  if (ldy < w->N) return fail(SHARQ_ERR_INVALID_ARG, "ldy=%lld < N=%lld", (long long)ldy, (long long)w->N);
  if (!aligned(y_dev, out_dtype == SHARQ_OUT_F32 ? 4 : 2)) return fail(SHARQ_ERR_INVALID_ARG, "output misaligned");
  if (!a->r_codes || !a->r_scales || !w->codes || !backbone_ok(a, a->n))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor buffers not set or not 16-byte aligned");
  if (!aligned(a->r_codes, 16) || !aligned(w->codes, 16) || !aligned(a->r_scales, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "operand buffers must be 16-byte aligned");
  const bool nv = a->fmt == SHARQ_FMT_NVFP4;
  const sharq_scale_view& vs = w->view[SHARQ_PATH_SPARSE];
  const sharq_scale_view& vd = w->view[SHARQ_PATH_DENSE];
  const int blk = nv ? 16 : 32;
  const int64_t nbld = (w->N + 15) / 16 * (nv ? 128 : 64);
  if (!vs.base || !vd.base || vs.block != blk || vd.block != blk || vs.ld != nbld || vd.ld != nbld ||
      !aligned(vs.base, 16) || !aligned(vd.base, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "weight scale views must be the tiled views of the weight's format (block %d, K-tile stride %lld)",
                blk, (long long)nbld);
  if (vs.base != vd.base)
    return fail(SHARQ_ERR_UNSUPPORTED, "the two paths must view the same packed scale array (distinct per-path scale arrays are not built)");
  s = check_device();
  if (s) return s;
  sharq::GemmArgs g{};
  g.s_codes = a->s_codes;
  g.s_meta = a->s_meta;
  g.s_scales = a->s_scales;
  g.r_codes = a->r_codes;
  g.r_scales = a->r_scales;
  g.w_codes = w->codes;
  g.w_scales_sparse = vs.base;
  g.w_scales_dense = vd.base;
  g.w_scales_ld = vs.ld;
  g.y = y_dev;
  g.ldy = ldy;
  g.M = a->M;
  g.N = w->N;
  g.K = (int)a->K;
  g.out_bf16 = out_dtype == SHARQ_OUT_BF16;
  g.resid = static_cast<const uint16_t*>(resid);
  g.ld_resid = ld_resid;
  g.a_blocks = (a->M + 15) / 16;
  g.xcd_bm = 0;
  g.seg = nullptr;
  g.pseg = nullptr;
  g.tprefix = nullptr;
  g.E = 0;
  g.g_s = g.g_r = g.g_w = nullptr;
  if (nv) {
    const sharq::NvActLayout la = sharq::nv_act_layout(a->M, a->K);
    const sharq::NvWeightLayout lw = sharq::nv_weight_layout(w->N, w->K);
    g.g_s = reinterpret_cast<const float*>(a->s_scales + la.g);
    g.g_r = reinterpret_cast<const float*>(a->r_scales + la.g);
    g.g_w = reinterpret_cast<const float*>(vs.base + lw.g);
  }
  hipError_t e = nv ? sharq::launch_linear_nv(g, static_cast<hipStream_t>(stream))
                 : a->n == 0 ? sharq::launch_linear_dense(g, static_cast<hipStream_t>(stream))
                             : sharq::launch_linear(g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return SHARQ_OK;
}

sharq_status sharq_linear(const sharq_act* a, const sharq_weight* w, void* y_dev, int64_t ldy, int32_t out_dtype,
                          void* stream) {
  g_err[0] = 0;
  return linear_impl(a, w, y_dev, ldy, out_dtype, nullptr, 0, stream);
}

sharq_status sharq_linear_residual(const sharq_act* a, const sharq_weight* w, const void* x_bf16_dev, int64_t ldx,
                                   void* y_bf16_dev, int64_t ldy, void* stream) {
  g_err[0] = 0;
  if (!a || !w) return fail(SHARQ_ERR_INVALID_ARG, "null descriptor");
  if (a->struct_size != sizeof(sharq_act) || w->struct_size != sizeof(sharq_weight))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor struct_size mismatch");
  if (a->fmt != SHARQ_FMT_MXFP4 || w->fmt != SHARQ_FMT_MXFP4)
    return fail(SHARQ_ERR_UNSUPPORTED, "the residual epilogue is built for MXFP4 layers");
  if (a->M > 0) {
    if (!x_bf16_dev) return fail(SHARQ_ERR_INVALID_ARG, "null residual pointer");
    if (ldx < w->N) return fail(SHARQ_ERR_INVALID_ARG, "ldx=%lld < N=%lld", (long long)ldx, (long long)w->N);
    if (!aligned(x_bf16_dev, 2)) return fail(SHARQ_ERR_INVALID_ARG, "residual misaligned");
  }
  return linear_impl(a, w, y_bf16_dev, ldy, SHARQ_OUT_BF16, x_bf16_dev, ldx, stream);
}

// sharq_linear_swiglu (H stored, next == nullptr) and sharq_linear_swiglu_prep
// (H prepared into *next)
static sharq_status swiglu_impl(const sharq_act* a, const sharq_weight* w, void* y_bf16_dev, int64_t ldy,
                                sharq_act* next, void* stream) {
  if (!a || !w) return fail(SHARQ_ERR_INVALID_ARG, "null descriptor");
  if (a->struct_size != sizeof(sharq_act) || w->struct_size != sizeof(sharq_weight))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor struct_size mismatch");
  if (a->layout_version != SHARQ_ABI_VERSION || w->layout_version != SHARQ_ABI_VERSION)
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor layout_version mismatch (not produced by this library?)");
  if (a->K != w->K) return fail(SHARQ_ERR_INVALID_ARG, "K mismatch: activation %lld, weight %lld", (long long)a->K, (long long)w->K);
  if (a->M < 0 || w->N <= 0 || a->K <= 0 || a->K % 32 || a->K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "bad shapes");
  if (w->N % 32) return fail(SHARQ_ERR_INVALID_ARG, "the gate/up weight needs N %% 32 == 0 (pairs of 16-row blocks), got %lld", (long long)w->N);
  if (a->fmt != w->fmt) return fail(SHARQ_ERR_INVALID_ARG, "activation and weight formats differ");
  sharq_status s = check_fmt(a->fmt);
  if (s) return s;
  if (a->fmt != SHARQ_FMT_MXFP4 || a->n != 2 || a->m != 4)
    return fail(SHARQ_ERR_UNSUPPORTED, "the SwiGLU epilogue is built for the 2:4 MXFP4 layer");
  const int64_t F = w->N / 2;
  if (next) {
    if (next->struct_size != sizeof(sharq_act)) return fail(SHARQ_ERR_INVALID_ARG, "output descriptor struct_size mismatch");
    if (F % 128) return fail(SHARQ_ERR_UNSUPPORTED, "preparing H in the epilogue needs N/2 %% 128 == 0, got %lld", (long long)F);
  }
  if (a->M > 0) {
    if (next) {
      if (!next->r_codes || !next->r_scales || !backbone_ok(next, 2) || !aligned(next->r_codes, 16) ||
          !aligned(next->r_scales, 16))
        return fail(SHARQ_ERR_INVALID_ARG, "output activation buffers not set or not 16-byte aligned");
    } else {
      if (!y_bf16_dev || !aligned(y_bf16_dev, 2)) return fail(SHARQ_ERR_INVALID_ARG, "output null or misaligned");
      if (ldy < F) return fail(SHARQ_ERR_INVALID_ARG, "ldy=%lld < N/2=%lld", (long long)ldy, (long long)F);
    }
  }
  if (a->M == 0) {
    if (next) {
      next->layout_version = SHARQ_ABI_VERSION;
      next->M = 0;
      next->K = F;
      next->n = 2;
      next->m = 4;
      next->fmt = SHARQ_FMT_MXFP4;
    }
    return SHARQ_OK;
  }
  if (!a->r_codes || !a->r_scales || !w->codes || !backbone_ok(a, a->n) || !aligned(a->r_codes, 16) ||
      !aligned(a->r_scales, 16) || !aligned(w->codes, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor buffers not set or not 16-byte aligned");
  const sharq_scale_view& vs = w->view[SHARQ_PATH_SPARSE];
  const sharq_scale_view& vd = w->view[SHARQ_PATH_DENSE];
  const int64_t nb64 = (w->N + 15) / 16 * 64;
  if (!vs.base || !vd.base || vs.block != 32 || vd.block != 32 || vs.ld != nb64 || vd.ld != nb64 ||
      !aligned(vs.base, 16) || !aligned(vd.base, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "weight scale views must be tiled MX views (block 32, K-tile stride NB*64)");
  if (vs.base != vd.base)
    return fail(SHARQ_ERR_UNSUPPORTED, "the two paths must view the same packed scale array");
  {
    // the SwiGLU epilogues run on the tiled kernel only, whose buffer offsets are 31-bit
    const uint64_t kb = (uint64_t)(a->K + 127) / 128, lim = 0x7FFFFFFFull;
    if ((uint64_t)(a->M + 15) / 16 * kb * 1024 >= lim || (uint64_t)(w->N + 15) / 16 * kb * 1024 >= lim)
      return fail(SHARQ_ERR_UNSUPPORTED, "the SwiGLU layer's operands past 2 GiB of codes (M=%lld, N=%lld, K=%lld)",
                  (long long)a->M, (long long)w->N, (long long)a->K);
  }
  s = check_device();
  if (s) return s;
  sharq::GemmArgs g{};
  g.s_codes = a->s_codes;
  g.s_meta = a->s_meta;
  g.s_scales = a->s_scales;
  g.r_codes = a->r_codes;
  g.r_scales = a->r_scales;
  g.w_codes = w->codes;
  g.w_scales_sparse = vs.base;
  g.w_scales_dense = vd.base;
  g.w_scales_ld = vs.ld;
  g.y = y_bf16_dev;
  g.ldy = ldy;
  g.M = a->M;
  g.N = w->N;
  g.K = (int)a->K;
  g.out_bf16 = 1;
  g.a_blocks = (a->M + 15) / 16;
  if (next) g.next = sharq::PrepOut{next->s_codes, next->s_meta, next->s_scales, next->r_codes, next->r_scales};
  hipError_t e = sharq::launch_linear_swiglu(g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "swiglu linear launch");
  if (next) {
    next->layout_version = SHARQ_ABI_VERSION;
    next->M = a->M;
    next->K = F;
    next->n = 2;
    next->m = 4;
    next->fmt = SHARQ_FMT_MXFP4;
  }
  return SHARQ_OK;
}

sharq_status sharq_linear_swiglu(const sharq_act* a, const sharq_weight* w, void* y_bf16_dev, int64_t ldy,
                                 void* stream) {
  g_err[0] = 0;
  return swiglu_impl(a, w, y_bf16_dev, ldy, nullptr, stream);
}

sharq_status sharq_linear_swiglu_prep(const sharq_act* a, const sharq_weight* w, sharq_act* next, void* stream) {
  g_err[0] = 0;
  if (!next) return fail(SHARQ_ERR_INVALID_ARG, "null output descriptor");
  return swiglu_impl(a, w, nullptr, 0, next, stream);
}

sharq_status sharq_linear_fused(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx,
                                const void* gamma_bf16_dev, float eps, int32_t n, int32_t m, int32_t fmt,
                                const sharq_weight* w, void* y_dev, int64_t ldy, int32_t out_dtype, void* stream) {
  g_err[0] = 0;
  if (!w) return fail(SHARQ_ERR_INVALID_ARG, "null weight descriptor");
  if (w->struct_size != sizeof(sharq_weight)) return fail(SHARQ_ERR_INVALID_ARG, "descriptor struct_size mismatch");
  if (w->layout_version != SHARQ_ABI_VERSION)
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor layout_version mismatch (not produced by this library?)");
  if (M < 0 || K <= 0 || K % 32) return fail(SHARQ_ERR_INVALID_ARG, "bad shape M=%lld K=%lld (K%%32 must be 0)", (long long)M, (long long)K);
  if (K != w->K) return fail(SHARQ_ERR_INVALID_ARG, "K mismatch: activation %lld, weight %lld", (long long)K, (long long)w->K);
  if (out_dtype != SHARQ_OUT_F32 && out_dtype != SHARQ_OUT_BF16) return fail(SHARQ_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dtype);
  sharq_status s = check_fmt(fmt);
  if (s) return s;
  if (fmt != w->fmt) return fail(SHARQ_ERR_INVALID_ARG, "activation and weight formats differ");
  if ((fmt != SHARQ_FMT_MXFP4 && fmt != SHARQ_FMT_NVFP4) || n != 2 || m != 4)
    return fail(SHARQ_ERR_UNSUPPORTED, "the one-launch layer is built for 2:4 MXFP4 and NVFP4-style layers");
  const bool nv = fmt == SHARQ_FMT_NVFP4;
  const size_t lds = nv ? sharq::nv_fused_layer_lds_bytes((int)K) : sharq::fused_layer_lds_bytes((int)K, gamma_bf16_dev != nullptr);
  if (M > 16 || K > 8192 || lds > 160 * 1024)
    return fail(SHARQ_ERR_UNSUPPORTED, "the one-launch layer takes M <= 16 and K <= 8192 (use sharq_prepare + sharq_linear)");
  if (M == 0) return SHARQ_OK;
  if (!x_bf16_dev || !y_dev) return fail(SHARQ_ERR_INVALID_ARG, "null pointer");
  if (ldx < K || ldx % 8 || ldx > (int64_t(1) << 26)) return fail(SHARQ_ERR_INVALID_ARG, "ldx=%lld must be >= K, a multiple of 8, <= 2^26", (long long)ldx);
  if (!aligned(x_bf16_dev, 16) || (gamma_bf16_dev && !aligned(gamma_bf16_dev, 16)))
    return fail(SHARQ_ERR_INVALID_ARG, "activation or gamma not 16-byte aligned");
  if (ldy < w->N) return fail(SHARQ_ERR_INVALID_ARG, "ldy=%lld < N=%lld", (long long)ldy, (long long)w->N);
  if (!aligned(y_dev, out_dtype == SHARQ_OUT_F32 ? 4 : 2)) return fail(SHARQ_ERR_INVALID_ARG, "output misaligned");
  if (!w->codes || !aligned(w->codes, 16)) return fail(SHARQ_ERR_INVALID_ARG, "weight codes null or misaligned");
  const sharq_scale_view& vs = w->view[SHARQ_PATH_SPARSE];
  const sharq_scale_view& vd = w->view[SHARQ_PATH_DENSE];
  const int blk = nv ? 16 : 32;
  const int64_t nbld = (w->N + 15) / 16 * (nv ? 128 : 64);
  if (!vs.base || !vd.base || vs.block != blk || vd.block != blk || vs.ld != nbld || vd.ld != nbld ||
      !aligned(vs.base, 16) || !aligned(vd.base, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "weight scale views must be the tiled views of the weight's format (block %d, K-tile stride %lld)",
                blk, (long long)nbld);
  if (vs.base != vd.base)
    return fail(SHARQ_ERR_UNSUPPORTED, "the two paths must view the same packed scale array");
  s = check_device();
  if (s) return s;
  sharq::GemmArgs g{};
  if (nv) g.g_w = reinterpret_cast<const float*>(vs.base + sharq::nv_weight_layout(w->N, w->K).g);
  g.w_codes = w->codes;
  g.w_scales_sparse = vs.base;
  g.w_scales_dense = vd.base;
  g.w_scales_ld = vs.ld;
  g.y = y_dev;
  g.ldy = ldy;
  g.M = M;
  g.N = w->N;
  g.K = (int)K;
  g.out_bf16 = out_dtype == SHARQ_OUT_BF16;
  g.a_blocks = 1;
  hipError_t e = nv ? sharq::launch_linear_fused_nv(static_cast<const uint16_t*>(x_bf16_dev), (int)M, (int)K, ldx,
                                                   static_cast<const uint16_t*>(gamma_bf16_dev), eps, g,
                                                   static_cast<hipStream_t>(stream))
                    : sharq::launch_linear_fused(static_cast<const uint16_t*>(x_bf16_dev), (int)M, (int)K, ldx,
                                                 static_cast<const uint16_t*>(gamma_bf16_dev), eps, g,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fused layer launch");
  return SHARQ_OK;
}

sharq_status sharq_rmsnorm(const void* x_bf16_dev, int64_t M, int64_t K, int64_t ldx, const void* gamma_bf16_dev,
                           float eps, void* y_bf16_dev, int64_t ldy, void* stream) {
  g_err[0] = 0;
  if (M < 0 || K <= 0 || K % 32 || K > 32768)
    return fail(SHARQ_ERR_INVALID_ARG, "bad shape M=%lld K=%lld (K%%32 == 0, K <= 32768)", (long long)M, (long long)K);
  if (M == 0) return SHARQ_OK;
  if (!x_bf16_dev || !gamma_bf16_dev || !y_bf16_dev) return fail(SHARQ_ERR_INVALID_ARG, "null pointer");
  if (ldx < K || ldx % 8 || ldy < K || ldy % 8 || ldx > (int64_t(1) << 26) || ldy > (int64_t(1) << 26))
    return fail(SHARQ_ERR_INVALID_ARG, "ldx=%lld / ldy=%lld must be >= K, multiples of 8, <= 2^26", (long long)ldx, (long long)ldy);
  if (!aligned(x_bf16_dev, 16) || !aligned(gamma_bf16_dev, 16) || !aligned(y_bf16_dev, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  sharq_status s = check_device();
  if (s) return s;
  hipError_t e = sharq::launch_rmsnorm_bf16(static_cast<const uint16_t*>(x_bf16_dev), M, (int)K, ldx,
                                            static_cast<const uint16_t*>(gamma_bf16_dev), eps,
                                            static_cast<uint16_t*>(y_bf16_dev), ldy, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  return SHARQ_OK;
}

sharq_status sharq_add_bf16_f32(const void* x_bf16_dev, const float* y_dev, void* out_bf16_dev, int64_t n,
                                void* stream) {
  g_err[0] = 0;
  if (n < 0) return fail(SHARQ_ERR_INVALID_ARG, "n=%lld", (long long)n);
  if (n == 0) return SHARQ_OK;
  if (!x_bf16_dev || !y_dev || !out_bf16_dev) return fail(SHARQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x_bf16_dev, 2) || !aligned(y_dev, 4) || !aligned(out_bf16_dev, 2)) return fail(SHARQ_ERR_INVALID_ARG, "misaligned");
  sharq_status s = check_device();
  if (s) return s;
  hipError_t e = sharq::launch_add_bf16_f32(static_cast<const uint16_t*>(x_bf16_dev), y_dev,
                                            static_cast<uint16_t*>(out_bf16_dev), n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "add launch");
  return SHARQ_OK;
}

sharq_status sharq_add_f32(const float* a_dev, const float* b_dev, float* y_dev, int64_t n, void* stream) {
  g_err[0] = 0;
  if (n < 0) return fail(SHARQ_ERR_INVALID_ARG, "n=%lld", (long long)n);
  if (n == 0) return SHARQ_OK;
  if (!a_dev || !b_dev || !y_dev) return fail(SHARQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(a_dev, 4) || !aligned(b_dev, 4) || !aligned(y_dev, 4)) return fail(SHARQ_ERR_INVALID_ARG, "misaligned");
  sharq_status s = check_device();
  if (s) return s;
  hipError_t e = sharq::launch_add_f32(a_dev, b_dev, y_dev, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "add launch");
  return SHARQ_OK;
}

sharq_status sharq_grouped_workspace_bytes(int64_t rows, int32_t E, int64_t K, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(SHARQ_ERR_INVALID_ARG, "null output");
  if (rows < 0 || E < 1 || E > 1024) return fail(SHARQ_ERR_INVALID_ARG, "bad rows=%lld or E=%d (1..1024)", (long long)rows, (int)E);
  if (K <= 0 || K % 32 || K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "bad K=%lld", (long long)K);
  *bytes = sharq::grouped_workspace_bytes(rows, E, (int)K);
  return SHARQ_OK;
}

}  // extern "C"

namespace {

// The grouped layer behind both entry points: with noalloc the workspace is
// the library's per-GPU scratch (ws_dev and ws_bytes unused).
// With `next` (the SwiGLU-prep form) the layer writes the down projection's
// prepared activation instead of Y (y_dev, ldy and out_dtype unused).
sharq_status linear_grouped_impl(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                 const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w, void* y_dev,
                                 int64_t ldy, int32_t out_dtype, void* ws_dev, size_t ws_bytes, bool noalloc,
                                 sharq_act* next, void* stream) {
  g_err[0] = 0;
  if (!a || !w) return fail(SHARQ_ERR_INVALID_ARG, "null descriptor");
  if (a->struct_size != sizeof(sharq_act) || w->struct_size != sizeof(sharq_weight))
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor struct_size mismatch");
  if (a->layout_version != SHARQ_ABI_VERSION || w->layout_version != SHARQ_ABI_VERSION)
    return fail(SHARQ_ERR_INVALID_ARG, "descriptor layout_version mismatch (not produced by this library?)");
  if (a->K != w->K) return fail(SHARQ_ERR_INVALID_ARG, "K mismatch: activation %lld, weight %lld", (long long)a->K, (long long)w->K);
  if (a->M < 0 || w->N <= 0 || a->K <= 0 || a->K % 32 || a->K > (1 << 30)) return fail(SHARQ_ERR_INVALID_ARG, "bad shapes");
  if (!next && out_dtype != SHARQ_OUT_F32 && out_dtype != SHARQ_OUT_BF16) return fail(SHARQ_ERR_INVALID_ARG, "unknown output dtype %d", (int)out_dtype);
  if (a->n != 2 || a->m != 4) return fail(SHARQ_ERR_UNSUPPORTED, "the grouped layer is built for the 2:4 pattern only");
  if (a->fmt != w->fmt) return fail(SHARQ_ERR_INVALID_ARG, "activation and weight formats differ");
  sharq_status s = check_fmt(a->fmt, false);
  if (s) return s;
  if (E < 1 || E > 1024) return fail(SHARQ_ERR_INVALID_ARG, "E=%d outside 1..1024", (int)E);
  if (w->N % E || (w->N / E) % 16)
    return fail(SHARQ_ERR_INVALID_ARG, "stacked weight N=%lld is not E=%d experts of a multiple of 16 rows", (long long)w->N, (int)E);
  const int64_t Ne = w->N / E;
  if (rows < 0) return fail(SHARQ_ERR_INVALID_ARG, "rows=%lld", (long long)rows);
  if (!row_index_dev && rows != a->M) return fail(SHARQ_ERR_INVALID_ARG, "without a row index the routed rows are the activation rows (rows=%lld, M=%lld)", (long long)rows, (long long)a->M);
  const int64_t F = Ne / 2;
  if (next) {
    if (next->struct_size != sizeof(sharq_act)) return fail(SHARQ_ERR_INVALID_ARG, "output descriptor struct_size mismatch");
    if (a->fmt != SHARQ_FMT_MXFP4) return fail(SHARQ_ERR_UNSUPPORTED, "the SwiGLU epilogue is built for the 2:4 MXFP4 layer");
    if (Ne % 32) return fail(SHARQ_ERR_INVALID_ARG, "each expert's gate/up rows need N_e %% 32 == 0 (pairs of 16-row blocks), got %lld", (long long)Ne);
    if (F % 128) return fail(SHARQ_ERR_UNSUPPORTED, "preparing H in the epilogue needs N_e/2 %% 128 == 0, got %lld", (long long)F);
  }
  if (rows == 0) {
    if (next) {
      next->layout_version = SHARQ_ABI_VERSION;
      next->M = 0;
      next->K = F;
      next->n = 2;
      next->m = 4;
      next->fmt = SHARQ_FMT_MXFP4;
    }
    return SHARQ_OK;
  }
  if (!seg_offsets_dev || !aligned(seg_offsets_dev, 8)) return fail(SHARQ_ERR_INVALID_ARG, "segment offsets null or misaligned");
  if (row_index_dev && !aligned(row_index_dev, 4)) return fail(SHARQ_ERR_INVALID_ARG, "row index misaligned");
  if (next) {
    if (!next->r_codes || !next->r_scales || !next->s_codes || !next->s_meta || !next->s_scales ||
        !aligned(next->r_codes, 16) || !aligned(next->r_scales, 16) || !aligned(next->s_codes, 16) ||
        !aligned(next->s_meta, 16) || !aligned(next->s_scales, 16))
      return fail(SHARQ_ERR_INVALID_ARG, "output activation buffers not set or not 16-byte aligned");
  } else {
    if (!y_dev) return fail(SHARQ_ERR_INVALID_ARG, "null output pointer");
    if (ldy < Ne) return fail(SHARQ_ERR_INVALID_ARG, "ldy=%lld < N_e=%lld", (long long)ldy, (long long)Ne);
    if (!aligned(y_dev, out_dtype == SHARQ_OUT_F32 ? 4 : 2)) return fail(SHARQ_ERR_INVALID_ARG, "output misaligned");
  }
  if (a->M > 0) {
    if (!a->s_codes || !a->s_meta || !a->s_scales || !a->r_codes || !a->r_scales)
      return fail(SHARQ_ERR_INVALID_ARG, "activation buffers not set");
    if (!aligned(a->s_codes, 16) || !aligned(a->s_meta, 16) || !aligned(a->r_codes, 16) ||
        !aligned(a->s_scales, 16) || !aligned(a->r_scales, 16))
      return fail(SHARQ_ERR_INVALID_ARG, "activation buffers must be 16-byte aligned");
  }
  if (!w->codes || !aligned(w->codes, 16)) return fail(SHARQ_ERR_INVALID_ARG, "weight codes null or misaligned");
  const sharq_scale_view& vs = w->view[SHARQ_PATH_SPARSE];
  const sharq_scale_view& vd = w->view[SHARQ_PATH_DENSE];
  const int64_t nb64 = (w->N + 15) / 16 * 64;
  if (!vs.base || !vd.base || vs.block != 32 || vd.block != 32 || vs.ld != nb64 || vd.ld != nb64 ||
      !aligned(vs.base, 16) || !aligned(vd.base, 16))
    return fail(SHARQ_ERR_INVALID_ARG, "weight scale views must be tiled MX views (block 32, K-tile stride NB*64)");
  if (vs.base != vd.base)
    return fail(SHARQ_ERR_UNSUPPORTED, "the two paths must view the same packed scale array (distinct per-path scale arrays are not built)");
  {
    // the tiled kernel addresses the source activation, the gathered one and
    // the weight with 31-bit buffer offsets
    const uint64_t kb = (uint64_t)(a->K + 127) / 128, lim = 0x7FFFFFFFull;
    const uint64_t src_blocks = (uint64_t)(a->M + 15) / 16, dst_blocks = (uint64_t)(rows + 15 * (int64_t)E + 15) / 16;
    const uint64_t w_blocks = (uint64_t)(w->N + 15) / 16;
    if (src_blocks * kb * 1024 >= lim || dst_blocks * kb * 1024 >= lim || w_blocks * kb * 1024 >= lim)
      return fail(SHARQ_ERR_UNSUPPORTED, "grouped operands past 2 GiB of codes (M=%lld, rows=%lld, N=%lld, K=%lld)",
                  (long long)a->M, (long long)rows, (long long)w->N, (long long)a->K);
  }
  const size_t need = sharq::grouped_workspace_bytes(rows, E, (int)a->K);
  if (noalloc) {
    if (need > sharq::kNoAllocScratchBytes)
      return fail(SHARQ_ERR_WORKSPACE, "this layer needs %zu bytes of workspace; the library's scratch holds %zu "
                  "(use sharq_linear_grouped with a caller workspace)", need, sharq::kNoAllocScratchBytes);
  } else if (!ws_dev || ws_bytes < need || !aligned(ws_dev, 256)) {
    return fail(SHARQ_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu", need, ws_bytes);
  }
  s = check_device();
  if (s) return s;
  if (noalloc) {
    hipError_t e = hipSuccess;
    ws_dev = sharq::noalloc_scratch(&e);
    if (!ws_dev) return hip_fail(e, "address of the library's scratch (hipGetSymbolAddress)");
  }
  sharq::GroupedArgs ga{};
  sharq::GemmArgs& g = ga.gemm;
  g.s_codes = a->s_codes;
  g.s_meta = a->s_meta;
  g.s_scales = a->s_scales;
  g.r_codes = a->r_codes;
  g.r_scales = a->r_scales;
  g.w_codes = w->codes;
  g.w_scales_sparse = vs.base;
  g.w_scales_dense = vd.base;
  g.w_scales_ld = vs.ld;
  g.y = y_dev;
  g.ldy = ldy;
  g.M = a->M;
  g.N = w->N;
  g.K = (int)a->K;
  g.out_bf16 = out_dtype == SHARQ_OUT_BF16;
  g.resid = nullptr;
  g.ld_resid = 0;
  g.a_blocks = (a->M + 15) / 16;
  g.xcd_bm = 0;
  g.seg = nullptr;
  g.pseg = nullptr;
  g.tprefix = nullptr;
  g.E = E;
  g.g_s = g.g_r = g.g_w = nullptr;
  ga.row_index = row_index_dev;
  ga.seg_in = seg_offsets_dev;
  ga.rows = rows;
  ga.src_blocks = (a->M + 15) / 16;
  ga.ws = static_cast<uint8_t*>(ws_dev);
  if (next) g.next = sharq::PrepOut{next->s_codes, next->s_meta, next->s_scales, next->r_codes, next->r_scales};
  hipError_t e = sharq::launch_linear_grouped(ga, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "grouped linear launch");
  if (next) {
    next->layout_version = SHARQ_ABI_VERSION;
    next->M = rows;
    next->K = F;
    next->n = 2;
    next->m = 4;
    next->fmt = SHARQ_FMT_MXFP4;
  }
  return SHARQ_OK;
}

}  // namespace

extern "C" {

sharq_status sharq_linear_grouped(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                  const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                  void* y_dev, int64_t ldy, int32_t out_dtype,
                                  void* ws_dev, size_t ws_bytes, void* stream) {
  return linear_grouped_impl(a, row_index_dev, rows, seg_offsets_dev, E, w, y_dev, ldy, out_dtype, ws_dev, ws_bytes,
                             false, nullptr, stream);
}

sharq_status sharq_linear_grouped_swiglu_prep(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                              const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                              sharq_act* next, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!next) {
    g_err[0] = 0;
    return fail(SHARQ_ERR_INVALID_ARG, "null output descriptor");
  }
  return linear_grouped_impl(a, row_index_dev, rows, seg_offsets_dev, E, w, nullptr, 0, SHARQ_OUT_BF16, ws_dev,
                             ws_bytes, false, next, stream);
}

sharq_status sharq_linear_grouped_noalloc(const sharq_act* a, const int32_t* row_index_dev, int64_t rows,
                                          const int64_t* seg_offsets_dev, int32_t E, const sharq_weight* w,
                                          void* y_dev, int64_t ldy, int32_t out_dtype, void* stream) {
  return linear_grouped_impl(a, row_index_dev, rows, seg_offsets_dev, E, w, y_dev, ldy, out_dtype, nullptr, 0, true,
                             nullptr, stream);
}

size_t sharq_noalloc_scratch_bytes(void) { return sharq::kNoAllocScratchBytes; }

}  // extern "C"
