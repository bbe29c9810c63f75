// api.hip - the extern "C" entry points of libmq.so.
//
// Argument checks run first and touch no HIP API, so every MQ_ERR_INVALID /
// MQ_ERR_SHAPE / MQ_ERR_ALIGN path works on a host without a GPU.  Only
// then is the current device looked up (once per device, cached) and the
// kernels queued on the caller's stream.  Nothing here allocates device
// memory or synchronises.
#include <mutex>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include "mq_internal.h"

namespace mq {

void log_launch(const char* kernel, unsigned grid, unsigned block, size_t lds, const char* fmt, ...) {
  static const bool on = [] {
    const char* v = getenv("MQ_LOG");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  if (!on) return;
  char shape[192];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(shape, sizeof shape, fmt, ap);
  va_end(ap);
  fprintf(stderr, "mq: %s grid=%u block=%u lds=%zu %s\n", kernel, grid, block, lds, shape);
}

}  // namespace mq

namespace {

thread_local char g_err[256] = "";

mq_status fail(mq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mq_status fail(mq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

mq_status ok() {
  g_err[0] = '\0';
  return MQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

mq_status check_dims(int64_t rows, int64_t cols, const char* rname, const char* cname) {
  if (rows < 1 || cols < 1) return fail(MQ_ERR_SHAPE, "%s=%lld and %s=%lld must be >= 1", rname, (long long)rows, cname, (long long)cols);
  if (rows > kMaxDim || cols > kMaxDim || rows * cols > ((int64_t)1 << 40))
    return fail(MQ_ERR_SHAPE, "%s=%lld x %s=%lld exceeds the supported size", rname, (long long)rows, cname, (long long)cols);
  return MQ_OK;
}

std::mutex g_dev_mu;
mq::DeviceInfo g_dev[64];

mq_status current_device(mq::DeviceInfo& out) {
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0) {
    (void)hipGetLastError();
    return fail(MQ_ERR_DEVICE, "no HIP device available");
  }
  if (d >= 64) return fail(MQ_ERR_DEVICE, "device index %d not supported", d);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  mq::DeviceInfo& di = g_dev[d];
  if (di.device != d) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MQ_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", d);
    }
    di.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    di.num_cu = prop.multiProcessorCount;
    di.device = d;
  }
  if (!di.ok) return fail(MQ_ERR_DEVICE, "device %d is not gfx950", d);
  out = di;
  return MQ_OK;
}

mq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MQ_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* mq_status_str(mq_status s) {
  switch (s) {
    case MQ_OK: return "MQ_OK";
    case MQ_ERR_INVALID: return "MQ_ERR_INVALID";
    case MQ_ERR_SHAPE: return "MQ_ERR_SHAPE";
    case MQ_ERR_ALIGN: return "MQ_ERR_ALIGN";
    case MQ_ERR_DEVICE: return "MQ_ERR_DEVICE";
    case MQ_ERR_LAUNCH: return "MQ_ERR_LAUNCH";
    default: return "MQ_ERR_UNKNOWN";
  }
}

const char* mq_last_error(void) { return g_err; }

const char* mq_version(void) { return "mq 0.1.0 (gfx950)"; }

mq_status mq_quantize_nvfp4(const void* x_bf16, int64_t rows, int64_t cols, const mq_nvfp4* out,
                            uint32_t flags, void* hip_stream) {
  if (!x_bf16 || !out) return fail(MQ_ERR_INVALID, "x_bf16 and out must not be NULL");
  if (!out->codes || !out->scales || !out->rec) return fail(MQ_ERR_INVALID, "out->codes, scales and rec must not be NULL");
  if (flags & ~(MQ_SCALE_GIVEN | MQ_SCALE_PARTIALS)) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if ((flags & MQ_SCALE_GIVEN) && (flags & MQ_SCALE_PARTIALS))
    return fail(MQ_ERR_INVALID, "MQ_SCALE_GIVEN and MQ_SCALE_PARTIALS are exclusive");
  if (mq_status s = check_dims(rows, cols, "rows", "cols")) return s;
  if (cols % 16) return fail(MQ_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (!aligned(x_bf16, 16) || !aligned(out->codes, 16) || !aligned(out->scales, 8) || !aligned(out->rec, 16))
    return fail(MQ_ERR_ALIGN, "x and codes need 16-byte, scales 8-byte, rec 16-byte alignment");
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  hipStream_t st = (hipStream_t)hip_stream;
  const bool given = flags & MQ_SCALE_GIVEN;
  const bool dynamic = !given && !(flags & MQ_SCALE_PARTIALS);
  const bool inline_amax = dynamic && rows * cols <= mq::kInlineAmaxElems;
  if (dynamic && !inline_amax && mq::quantize_resident_pays(rows * cols, dev))
    return launched(mq::launch_quantize_resident(x_bf16, rows * cols, out->codes, out->scales, out->rec, dev, st),
                    "quantize");
  if (dynamic && !inline_amax) {
    hipError_t e = mq::launch_amax(x_bf16, rows * cols, out->rec, dev, st);
    if (e != hipSuccess) return launched(e, "amax");
  }
  return launched(mq::launch_quantize(x_bf16, rows * cols, out->codes, out->scales, out->rec, given, dev, st,
                                      inline_amax),
                  "quantize");
}

mq_status mq_gemm_nvfp4_prefill_grouped(const mq_nvfp4* a, const void* a_bf16, int32_t n_group,
                                        const mq_nvfp4* w, void* const* c, const int64_t* N, int64_t M,
                                        int64_t K, uint32_t flags, void* hip_stream) {
  const uint32_t known = MQ_OUT_F32 | MQ_A_FUSED_BF16 | MQ_SCALE_GIVEN | MQ_SCALE_PARTIALS;
  if (flags & ~known) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  const bool fused = flags & MQ_A_FUSED_BF16;
  if ((flags & (MQ_SCALE_GIVEN | MQ_SCALE_PARTIALS)) && !fused)
    return fail(MQ_ERR_INVALID, "MQ_SCALE_GIVEN and MQ_SCALE_PARTIALS need MQ_A_FUSED_BF16");
  if ((flags & MQ_SCALE_GIVEN) && (flags & MQ_SCALE_PARTIALS))
    return fail(MQ_ERR_INVALID, "MQ_SCALE_GIVEN and MQ_SCALE_PARTIALS are exclusive");
  if (n_group < 1 || n_group > MQ_MAX_GROUP)
    return fail(MQ_ERR_INVALID, "n_group=%d must be in 1..%d", (int)n_group, MQ_MAX_GROUP);
  if (!a || !w || !c || !N) return fail(MQ_ERR_INVALID, "a, w, c and N must not be NULL");
  if (!a->rec) return fail(MQ_ERR_INVALID, "a->rec must not be NULL");
  if (fused) {
    if (!a_bf16) return fail(MQ_ERR_INVALID, "MQ_A_FUSED_BF16 needs a_bf16");
    if (!a->codes != !a->scales)
      return fail(MQ_ERR_INVALID, "with MQ_A_FUSED_BF16 give both a->codes and a->scales, or neither");
  } else {
    if (a_bf16) return fail(MQ_ERR_INVALID, "a_bf16 must be NULL without MQ_A_FUSED_BF16");
    if (!a->codes || !a->scales) return fail(MQ_ERR_INVALID, "a->codes and a->scales must not be NULL");
  }
  if (mq_status s = check_dims(M, K, "M", "K")) return s;
  if (K % 16) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (!aligned(a->rec, 16)) return fail(MQ_ERR_ALIGN, "a->rec needs 16-byte alignment");
  if (fused && !aligned(a_bf16, 16)) return fail(MQ_ERR_ALIGN, "a_bf16 needs 16-byte alignment");
  if ((!fused || a->codes) && (!aligned(a->codes, 16) || !aligned(a->scales, 8)))
    return fail(MQ_ERR_ALIGN, "a->codes need 16-byte, a->scales 8-byte alignment");
  mq::GemmWeight gw[MQ_MAX_GROUP];
  int64_t ncols = 0;
  for (int g = 0; g < n_group; ++g) {
    const mq_nvfp4& wg = w[g];
    if (!wg.codes || !wg.scales || !wg.rec || !c[g])
      return fail(MQ_ERR_INVALID, "group %d: w codes, scales, rec and c must not be NULL", g);
    if (mq_status s = check_dims(N[g], K, "N", "K")) return s;
    if (M * N[g] > ((int64_t)1 << 40)) return fail(MQ_ERR_SHAPE, "group %d: M*N too large", g);
    if (!aligned(wg.codes, 16) || !aligned(wg.scales, 8) || !aligned(wg.rec, 16) || !aligned(c[g], 16))
      return fail(MQ_ERR_ALIGN, "group %d: codes and c need 16-byte, scales 8-byte, rec 16-byte alignment", g);
    ncols += N[g];
    gw[g] = mq::GemmWeight{wg.codes, wg.scales, wg.rec, c[g], N[g]};
  }
  if (ncols > kMaxDim) return fail(MQ_ERR_SHAPE, "the groups' N add up to more than %lld", (long long)kMaxDim);
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  hipStream_t st = (hipStream_t)hip_stream;
  const bool given = flags & MQ_SCALE_GIVEN;
  const bool dynamic = fused && !given && !(flags & MQ_SCALE_PARTIALS);
  // the per-tile fused form on a small A takes the maximum inside the GEMM
  // (the quantize-once form's tiled kernels read partial maxima; the small-
  // problem kernel takes the maximum itself in every A form)
  const bool inline_amax =
      dynamic && M * K <= mq::kInlineAmaxElems && (!a->codes || mq::gemm_small_rows(M));
  if (dynamic && !inline_amax) {
    hipError_t e = mq::launch_amax(a_bf16, M * K, a->rec, dev, st);
    if (e != hipSuccess) return launched(e, "amax");
  }
  const mq::GemmOperandA A{fused ? nullptr : a->codes, fused ? nullptr : a->scales, fused ? a_bf16 : nullptr,
                           a->rec, given, fused ? a->codes : nullptr, fused ? a->scales : nullptr,
                           inline_amax};
  return launched(mq::launch_gemm(A, gw, n_group, M, K, flags & MQ_OUT_F32, dev, st), fused ? "gemm_fused" : "gemm");
}

mq_status mq_gemm_nvfp4_prefill(const mq_nvfp4* a, const void* a_bf16, const mq_nvfp4* w, void* c,
                                int64_t M, int64_t N, int64_t K, uint32_t flags, void* hip_stream) {
  if (!w || !c) return fail(MQ_ERR_INVALID, "a, w and c must not be NULL");
  return mq_gemm_nvfp4_prefill_grouped(a, a_bf16, 1, w, &c, &N, M, K, flags, hip_stream);
}

mq_status mq_gemv_bf16_decode_grouped(const void* x_bf16, int32_t n_group, const void* const* w_bf16,
                                      void* const* y_bf16, const int64_t* N, int64_t M, int64_t K, uint32_t flags,
                                      void* hip_stream) {
  if (flags) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if (n_group < 1 || n_group > MQ_MAX_GROUP)
    return fail(MQ_ERR_INVALID, "n_group=%d must be in 1..%d", (int)n_group, MQ_MAX_GROUP);
  if (!x_bf16 || !w_bf16 || !y_bf16 || !N) return fail(MQ_ERR_INVALID, "x, w, y and N must not be NULL");
  if (M < 1 || M > 32) return fail(MQ_ERR_SHAPE, "M=%lld must be in 1..32", (long long)M);
  if (K < 1 || K > kMaxDim) return fail(MQ_ERR_SHAPE, "K=%lld out of range", (long long)K);
  if (K % 16) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (!aligned(x_bf16, 16)) return fail(MQ_ERR_ALIGN, "x needs 16-byte alignment");
  mq::GemvWeight gw[MQ_MAX_GROUP];
  int64_t nrows = 0;
  for (int g = 0; g < n_group; ++g) {
    if (!w_bf16[g] || !y_bf16[g]) return fail(MQ_ERR_INVALID, "group %d: w and y must not be NULL", g);
    if (mq_status s = check_dims(N[g], K, "N", "K")) return s;
    if (!aligned(w_bf16[g], 16) || !aligned(y_bf16[g], 2))
      return fail(MQ_ERR_ALIGN, "group %d: w needs 16-byte alignment, y 2-byte", g);
    nrows += N[g];
    gw[g] = mq::GemvWeight{w_bf16[g], y_bf16[g], N[g]};
  }
  if (nrows > kMaxDim) return fail(MQ_ERR_SHAPE, "the groups' N add up to more than %lld", (long long)kMaxDim);
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  return launched(mq::launch_gemv_grouped(x_bf16, gw, n_group, M, K, dev, (hipStream_t)hip_stream), "gemv");
}

mq_status mq_gemv_bf16_decode(const void* x_bf16, const void* w_bf16, void* y_bf16, int64_t M, int64_t N,
                              int64_t K, uint32_t flags, void* hip_stream) {
  if (!w_bf16 || !y_bf16) return fail(MQ_ERR_INVALID, "x, w and y must not be NULL");
  return mq_gemv_bf16_decode_grouped(x_bf16, 1, &w_bf16, &y_bf16, &N, M, K, flags, hip_stream);
}

mq_status mq_gemv_nvfp4_decode(const mq_nvfp4* x, const mq_nvfp4* w, void* y_bf16, int64_t M, int64_t N,
                               int64_t K, uint32_t flags, void* hip_stream) {
  if (flags) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if (!x || !w || !y_bf16) return fail(MQ_ERR_INVALID, "x, w and y must not be NULL");
  if (!x->codes || !x->scales || !x->rec || !w->codes || !w->scales || !w->rec)
    return fail(MQ_ERR_INVALID, "x and w codes, scales and rec must not be NULL");
  if (M < 1 || M > 32) return fail(MQ_ERR_SHAPE, "M=%lld must be in 1..32", (long long)M);
  if (mq_status s = check_dims(N, K, "N", "K")) return s;
  if (K % 16) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (!aligned(x->codes, 16) || !aligned(w->codes, 16) || !aligned(x->scales, 8) || !aligned(w->scales, 8) ||
      !aligned(x->rec, 16) || !aligned(w->rec, 16) || !aligned(y_bf16, 2))
    return fail(MQ_ERR_ALIGN, "codes need 16-byte, scales 8-byte, rec 16-byte, y 2-byte alignment");
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  const mq::GemvNvfp4Args a{x->codes, x->scales, x->rec, w->codes, w->scales, w->rec, y_bf16, M, N, K};
  return launched(mq::launch_gemv_nvfp4(a, (hipStream_t)hip_stream), "gemv_nvfp4");
}

mq_status mq_rmsnorm_amax(const void* x_bf16, const void* gamma_bf16, void* y_bf16, mq_scale_rec* rec,
                          int64_t rows, int64_t cols, float eps, uint32_t flags, void* hip_stream) {
  if (flags) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if (!x_bf16 || !gamma_bf16 || !y_bf16 || !rec) return fail(MQ_ERR_INVALID, "x, gamma, y and rec must not be NULL");
  if (mq_status s = check_dims(rows, cols, "rows", "cols")) return s;
  if (cols % 16) return fail(MQ_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(MQ_ERR_INVALID, "eps must be finite and >= 0");
  if (!aligned(x_bf16, 16) || !aligned(gamma_bf16, 16) || !aligned(y_bf16, 16) || !aligned(rec, 16))
    return fail(MQ_ERR_ALIGN, "x, gamma, y and rec need 16-byte alignment");
  if (x_bf16 == y_bf16) return fail(MQ_ERR_INVALID, "y must not alias x");
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  return launched(mq::launch_rmsnorm_amax(x_bf16, gamma_bf16, y_bf16, rows, cols, eps, rec, dev,
                                          (hipStream_t)hip_stream),
                  "rmsnorm_amax");
}

mq_status mq_rmsnorm_quantize_nvfp4(const void* x_bf16, const void* gamma_bf16, int64_t rows, int64_t cols,
                                    float eps, const mq_nvfp4* out, uint32_t flags, void* hip_stream) {
  if (flags) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if (!x_bf16 || !gamma_bf16 || !out) return fail(MQ_ERR_INVALID, "x, gamma and out must not be NULL");
  if (!out->codes || !out->scales || !out->rec)
    return fail(MQ_ERR_INVALID, "out->codes, scales and rec must not be NULL");
  if (mq_status s = check_dims(rows, cols, "rows", "cols")) return s;
  if (cols % 16) return fail(MQ_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(MQ_ERR_INVALID, "eps must be finite and >= 0");
  if (!aligned(x_bf16, 16) || !aligned(gamma_bf16, 16) || !aligned(out->codes, 16) || !aligned(out->scales, 8) ||
      !aligned(out->rec, 16))
    return fail(MQ_ERR_ALIGN, "x, gamma and codes need 16-byte, scales 8-byte, rec 16-byte alignment");
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  return launched(mq::launch_rmsnorm_quantize(x_bf16, gamma_bf16, rows, cols, eps, out->codes, out->scales, out->rec,
                                              dev, (hipStream_t)hip_stream),
                  "rmsnorm_quantize");
}

mq_status mq_swiglu_amax(const void* a_bf16, const void* b_bf16, void* y_bf16, mq_scale_rec* rec, int64_t rows,
                         int64_t cols, uint32_t flags, void* hip_stream) {
  if (flags) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if (!a_bf16 || !b_bf16 || !y_bf16 || !rec) return fail(MQ_ERR_INVALID, "a, b, y and rec must not be NULL");
  if (mq_status s = check_dims(rows, cols, "rows", "cols")) return s;
  if (cols % 16) return fail(MQ_ERR_SHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (!aligned(a_bf16, 16) || !aligned(b_bf16, 16) || !aligned(y_bf16, 16) || !aligned(rec, 16))
    return fail(MQ_ERR_ALIGN, "a, b, y and rec need 16-byte alignment");
  if (y_bf16 == a_bf16 || y_bf16 == b_bf16) return fail(MQ_ERR_INVALID, "y must not alias a or b");
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  return launched(mq::launch_swiglu_amax(a_bf16, b_bf16, y_bf16, rows * cols, rec, dev, (hipStream_t)hip_stream),
                  "swiglu_amax");
}

// ------------------------------------------------------- phase-aware linear --

int32_t mq_linear_path(const mq_linear* L, int64_t M, uint32_t flags) {
  if (!L || M < 1) return 0;
  if (L->prefill_min_rows < 1 || L->prefill_min_rows > 33) return 0;
  const uint32_t phase = flags & (MQ_PHASE_PREFILL | MQ_PHASE_DECODE);
  if (phase == (MQ_PHASE_PREFILL | MQ_PHASE_DECODE)) return 0;
  const bool prefill = phase == MQ_PHASE_PREFILL || (phase == 0 && M >= L->prefill_min_rows);
  if (prefill) return MQ_PATH_PREFILL_NVFP4;
  return M <= 32 ? MQ_PATH_DECODE_BF16 : 0;
}

}  // extern "C"

namespace {

// Checks of the weight side of a linear, shared by prepare and forward.
mq_status check_linear(const mq_linear* L) {
  if (!L) return fail(MQ_ERR_INVALID, "L must not be NULL");
  if (!L->w_bf16 || !L->w_nvfp4.codes || !L->w_nvfp4.scales || !L->w_nvfp4.rec)
    return fail(MQ_ERR_INVALID, "L->w_bf16 and L->w_nvfp4 codes, scales and rec must not be NULL");
  if (mq_status s = check_dims(L->N, L->K, "N", "K")) return s;
  if (L->K % 16) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)L->K);
  if (!aligned(L->w_bf16, 16) || !aligned(L->w_nvfp4.codes, 16) || !aligned(L->w_nvfp4.scales, 8) ||
      !aligned(L->w_nvfp4.rec, 16))
    return fail(MQ_ERR_ALIGN, "w_bf16 and codes need 16-byte, scales 8-byte, rec 16-byte alignment");
  return MQ_OK;
}

}  // namespace

extern "C" {

mq_status mq_linear_prepare(const mq_linear* L, void* hip_stream) {
  if (mq_status s = check_linear(L)) return s;
  return mq_quantize_nvfp4(L->w_bf16, L->N, L->K, &L->w_nvfp4, MQ_SCALE_DYNAMIC, hip_stream);
}

mq_status mq_linear_forward(const mq_linear* L, const void* x_bf16, int64_t M, const mq_nvfp4* a_work,
                            void* y_bf16, uint32_t flags, void* hip_stream) {
  const uint32_t known = MQ_PHASE_PREFILL | MQ_PHASE_DECODE | MQ_A_FUSED_BF16 | MQ_SCALE_PARTIALS;
  if (flags & ~known) return fail(MQ_ERR_INVALID, "unknown flags 0x%x", flags);
  if ((flags & MQ_PHASE_PREFILL) && (flags & MQ_PHASE_DECODE))
    return fail(MQ_ERR_INVALID, "MQ_PHASE_PREFILL and MQ_PHASE_DECODE are exclusive");
  if (mq_status s = check_linear(L)) return s;
  if (L->prefill_min_rows < 1 || L->prefill_min_rows > 33)
    return fail(MQ_ERR_INVALID, "prefill_min_rows=%lld must be in 1..33", (long long)L->prefill_min_rows);
  if (!x_bf16 || !y_bf16) return fail(MQ_ERR_INVALID, "x and y must not be NULL");
  if (M < 1 || M > kMaxDim) return fail(MQ_ERR_SHAPE, "M=%lld out of range", (long long)M);
  const int32_t path = mq_linear_path(L, M, flags);
  if (path == 0) return fail(MQ_ERR_SHAPE, "M=%lld: a decode call takes 1..32 rows", (long long)M);
  if (!aligned(x_bf16, 16)) return fail(MQ_ERR_ALIGN, "x needs 16-byte alignment");
  if (path == MQ_PATH_DECODE_BF16) {
    if (!aligned(y_bf16, 2)) return fail(MQ_ERR_ALIGN, "y needs 2-byte alignment");
    return mq_gemv_bf16_decode(x_bf16, L->w_bf16, y_bf16, M, L->N, L->K, 0, hip_stream);
  }
  // prefill: every check of both launches before the first is queued
  const bool fused = flags & MQ_A_FUSED_BF16;
  if (!a_work || !a_work->rec) return fail(MQ_ERR_INVALID, "a prefill call needs a_work with rec");
  if (!fused && (!a_work->codes || !a_work->scales))
    return fail(MQ_ERR_INVALID, "a_work->codes and a_work->scales must not be NULL");
  if (!aligned(a_work->rec, 16) || (!fused && (!aligned(a_work->codes, 16) || !aligned(a_work->scales, 8))))
    return fail(MQ_ERR_ALIGN, "a_work: codes need 16-byte, scales 8-byte, rec 16-byte alignment");
  if (!aligned(y_bf16, 16)) return fail(MQ_ERR_ALIGN, "y needs 16-byte alignment on the prefill path");
  if (M * L->K > ((int64_t)1 << 40) || M * L->N > ((int64_t)1 << 40))
    return fail(MQ_ERR_SHAPE, "M=%lld exceeds the supported size", (long long)M);
  const uint32_t scale = flags & MQ_SCALE_PARTIALS;
  if (fused)
    return mq_gemm_nvfp4_prefill(a_work, x_bf16, &L->w_nvfp4, y_bf16, M, L->N, L->K, MQ_A_FUSED_BF16 | scale,
                                 hip_stream);
  if (mq_status s = mq_quantize_nvfp4(x_bf16, M, L->K, a_work, scale, hip_stream)) return s;
  return mq_gemm_nvfp4_prefill(a_work, nullptr, &L->w_nvfp4, y_bf16, M, L->N, L->K, 0, hip_stream);
}

}  // extern "C"

// ------------------------------------------------------ allocation-free call --
//
// Scratch for the quantized activation of mq_gemm_nvfp4_prefill_fused_noalloc:
// one scale record, then A's codes and scale bytes, at fixed 256-byte
// aligned offsets.  It is a module global: each device the library runs on
// holds its own copy, for the life of the process.  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// handed to kernels.

namespace {

constexpr size_t kScratchRec = 0;
constexpr size_t kScratchCodes = 4096;
constexpr size_t kScratchScales = kScratchCodes + (size_t)MQ_NOALLOC_MAX_ELEMS / 2;
constexpr size_t kScratchBytes = kScratchScales + (size_t)MQ_NOALLOC_MAX_ELEMS / 16;
static_assert(sizeof(mq_scale_rec) <= kScratchCodes - kScratchRec, "record slot");
static_assert(kScratchScales % 256 == 0 && kScratchBytes % 256 == 0, "scratch layout");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

uint8_t* g_scratch[64] = {};  // device address of `scratch`, per device (under g_dev_mu)

mq_status scratch_address(int device, uint8_t*& out) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(MQ_ERR_DEVICE, "device %d: no address for the scratch buffer (%s)", device, hipGetErrorString(e));
    }
    g_scratch[device] = (uint8_t*)p;
  }
  out = g_scratch[device];
  return MQ_OK;
}

}  // namespace

extern "C" {

mq_status mq_gemm_nvfp4_prefill_fused_noalloc(const void* a_bf16, const mq_nvfp4* w, void* c, int64_t M,
                                              int64_t N, int64_t K, uint32_t flags, void* hip_stream) {
  if (flags & ~(MQ_OUT_F32 | MQ_A_FUSED_BF16)) return fail(MQ_ERR_INVALID, "unknown or unsupported flags 0x%x", flags);
  if (!a_bf16 || !w || !c) return fail(MQ_ERR_INVALID, "a_bf16, w and c must not be NULL");
  if (mq_status s = check_dims(M, K, "M", "K")) return s;
  if (K % 16) return fail(MQ_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (M * K > (int64_t)MQ_NOALLOC_MAX_ELEMS)
    return fail(MQ_ERR_SHAPE, "M*K=%lld exceeds the scratch buffer's %lld elements", (long long)(M * K),
                (long long)MQ_NOALLOC_MAX_ELEMS);
  mq::DeviceInfo dev;
  if (mq_status s = current_device(dev)) return s;
  uint8_t* base = nullptr;
  if (mq_status s = scratch_address(dev.device, base)) return s;
  const mq_nvfp4 a{base + kScratchCodes, base + kScratchScales, (mq_scale_rec*)(base + kScratchRec)};
  return mq_gemm_nvfp4_prefill(&a, a_bf16, w, c, M, N, K, flags | MQ_A_FUSED_BF16, hip_stream);
}

}  // extern "C"
