// C-ABI entry points of include/q4f16.h: argument validation, plan choice and
// launches.  Validation runs on the host before any HIP call, so argument errors
// never enqueue work (and can be checked on a machine without a GPU).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "q4f16.h"
#include "q4_internal.h"
#include "q4_step.h"
#include <algorithm>
#include <cstring>

#include "q4_step_mfma.h"
#include "q4_formats.h"
#include "q4_fused.h"
#include <initializer_list>
#include <utility>

namespace {

thread_local std::string g_error;

int ok() {
  g_error.clear();
  return Q4_OK;
}

__attribute__((format(printf, 2, 3))) int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int device_error(hipError_t e, const char* what) {
  return fail(Q4_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int64_t N, int64_t K) {
  if (N < 1) return fail(Q4_ERR_SHAPE, "N = %lld: must be >= 1", (long long)N);
  if (K < 32 || K % 32) return fail(Q4_ERR_SHAPE, "K = %lld: must be a positive multiple of 32",
                                    (long long)K);
  if (N > (int64_t)INT32_MAX || K / 32 > (int64_t)INT32_MAX / 8)
    return fail(Q4_ERR_UNSUPPORTED, "N = %lld, K = %lld: too large", (long long)N, (long long)K);
  if (N * (K / 32) > ((int64_t)1 << 40))
    return fail(Q4_ERR_UNSUPPORTED, "N * K / 32 = %lld: too large", (long long)(N * (K / 32)));
  return Q4_OK;
}

// Validate one GEMV's tensors.  `what` names the call for the error text.
// x_cols: elements per row of x (K, or 2K when x holds gate | up).
int check_gemv(const char* what, const uint32_t* words, const uint16_t* scales,
               const uint16_t* x, const uint16_t* y, int64_t M, int64_t N, int64_t K,
               int64_t x_cols, uint32_t format = 0, const uint16_t* biases = nullptr) {
  if (!words) return fail(Q4_ERR_NULL, "%s: words is NULL", what);
  if (!scales) return fail(Q4_ERR_NULL, "%s: scales is NULL", what);
  if (!x) return fail(Q4_ERR_NULL, "%s: x is NULL", what);
  if (!y) return fail(Q4_ERR_NULL, "%s: y is NULL", what);
  if (M < 1 || M > q4::kMaxM)
    return fail(Q4_ERR_SHAPE, "%s: M = %lld: must be in [1, %d]", what, (long long)M, q4::kMaxM);
  int rc = check_shape(N, K);
  if (rc) return fail(rc, "%s: %s", what, g_error.c_str());
  const bool q3 = format == Q4_FMT_Q3F16_1;
  if (!aligned(words, q3 ? 4 : 16))
    return fail(Q4_ERR_ALIGN, "%s: words %p not %d-byte aligned", what, (const void*)words,
                q3 ? 4 : 16);
  if (!aligned(x, 16)) return fail(Q4_ERR_ALIGN, "%s: x %p not 16-byte aligned", what,
                                   (const void*)x);
  if (!aligned(scales, 2)) return fail(Q4_ERR_ALIGN, "%s: scales %p not 2-byte aligned", what,
                                       (const void*)scales);
  if (!aligned(y, 2)) return fail(Q4_ERR_ALIGN, "%s: y %p not 2-byte aligned", what,
                                  (const void*)y);
  // the output must not overlap an input
  const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uintptr_t)(2 * M * N);
  auto overlaps = [&](const void* p, int64_t bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)bytes;
    return a0 < y1 && y0 < a1;
  };
  // scales (and the affine biases): 2 bytes per 32 weights, or per 64 (affine)
  const bool aff = format == Q4_FMT_AF4_G64 || format == Q4_FMT_AF4_G64_F16;
  const int64_t sbytes = aff ? N * K / 32 : N * K / 16;
  if (biases && !aligned(biases, 2))
    return fail(Q4_ERR_ALIGN, "%s: biases %p not 2-byte aligned", what, (const void*)biases);
  if (overlaps(words, q3 ? N * K / 32 * 12 : N * K / 2) || overlaps(scales, sbytes) ||
      (biases && overlaps(biases, sbytes)) || overlaps(x, 2 * M * x_cols))
    return fail(Q4_ERR_SHAPE, "%s: y overlaps an input", what);
  return Q4_OK;
}

int check_ws(const char* what, void* ws, size_t have, size_t need) {
  if (need == 0) return Q4_OK;
  if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: needs %zu workspace bytes, ws is NULL", what, need);
  if (have < need)
    return fail(Q4_ERR_WORKSPACE, "%s: needs %zu workspace bytes, got %zu", what, need, have);
  if (!aligned(ws, 16)) return fail(Q4_ERR_ALIGN, "%s: ws %p not 16-byte aligned", what, ws);
  return Q4_OK;
}

std::mutex g_dev_mutex;
q4::DeviceInfo g_dev[64];

}  // namespace

namespace q4 {

int api_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int api_ok() { return ok(); }

const DeviceInfo* device_info() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceInfo& d = g_dev[dev];
  if (d.id < 0) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    d.cus = cus;
    d.lds_per_block = (size_t)lds;
    d.id = dev;
  }
  return &d;
}

}  // namespace q4

extern "C" {

const char* q4_status_str(int status) {
  switch (status) {
    case Q4_OK: return "Q4_OK";
    case Q4_ERR_NULL: return "Q4_ERR_NULL";
    case Q4_ERR_SHAPE: return "Q4_ERR_SHAPE";
    case Q4_ERR_ALIGN: return "Q4_ERR_ALIGN";
    case Q4_ERR_WORKSPACE: return "Q4_ERR_WORKSPACE";
    case Q4_ERR_DEVICE: return "Q4_ERR_DEVICE";
    case Q4_ERR_UNSUPPORTED: return "Q4_ERR_UNSUPPORTED";
    case Q4_ERR_TIMEOUT: return "Q4_ERR_TIMEOUT";
    default: return "Q4_ERR_UNKNOWN";
  }
}

const char* q4_last_error_detail(void) { return g_error.c_str(); }

const char* q4_last_error(void) { return g_error.c_str(); }

int q4_version(void) { return 200; }

int q4_pack(const uint8_t* codes, uint32_t* words, int64_t N, int64_t K, q4_stream_t stream) {
  if (!codes) return fail(Q4_ERR_NULL, "q4_pack: codes is NULL");
  if (!words) return fail(Q4_ERR_NULL, "q4_pack: words is NULL");
  if (int rc = check_shape(N, K)) return fail(rc, "q4_pack: %s", g_error.c_str());
  if (!aligned(words, 16)) return fail(Q4_ERR_ALIGN, "q4_pack: words not 16-byte aligned");
  hipError_t e = q4::launch_pack(codes, words, N, K, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_pack");
}

int q4_unpack(const uint32_t* words, uint8_t* codes, int64_t N, int64_t K, q4_stream_t stream) {
  if (!words) return fail(Q4_ERR_NULL, "q4_unpack: words is NULL");
  if (!codes) return fail(Q4_ERR_NULL, "q4_unpack: codes is NULL");
  if (int rc = check_shape(N, K)) return fail(rc, "q4_unpack: %s", g_error.c_str());
  if (!aligned(words, 16)) return fail(Q4_ERR_ALIGN, "q4_unpack: words not 16-byte aligned");
  hipError_t e = q4::launch_unpack(words, codes, N, K, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_unpack");
}

size_t q4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > q4::kMaxM || N < 1 || K < 32 || K % 32) return 0;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return 0;
  return q4::plan_auto(*d, M, N, K).ws_bytes;
}

size_t q4_splitk_workspace_bytes(int64_t M, int64_t N, int64_t splits) {
  if (M < 1 || M > q4::kMaxM || N < 1 || splits < 2) return 0;
  return (size_t)4 * (size_t)splits * (size_t)M * (size_t)N;
}

}  // extern "C"

namespace q4 {

int gemv_validate(const char* what, const uint32_t* words, const uint16_t* scales,
                  const uint16_t* x, const uint16_t* y, int64_t M, int64_t N, int64_t K,
                  int64_t x_cols, uint32_t format, const uint16_t* biases) {
  return check_gemv(what, words, scales, x, y, M, N, K, x_cols ? x_cols : K, format, biases);
}

int ws_validate(const char* what, void* ws, size_t have, size_t need) {
  return check_ws(what, ws, have, need);
}

int device_fail(hipError_t e, const char* what) { return device_error(e, what); }

int gemv_common(const char* what, const uint32_t* words, const uint16_t* scales,
                const uint16_t* x, uint16_t* y, int64_t M, int64_t N, int64_t K,
                int64_t splits, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_gemv(what, words, scales, x, y, M, N, K, K)) return rc;
  if (splits != 0 && (splits < 1 || splits > q4::kMaxSplits || splits > K / 32))
    return fail(Q4_ERR_SHAPE, "%s: splits = %lld: must be in [1, min(64, K/32 = %lld)]", what,
                (long long)splits, (long long)(K / 32));
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  q4::GemvPlan p = splits == 0 ? q4::plan_auto(*d, M, N, K)
                               : q4::plan_splits(*d, M, N, K, (int)splits);
  const int64_t gmax = (K / 32 + p.splits - 1) / p.splits;
  if (gmax > q4::max_groups_per_slice(*d, M))
    return fail(Q4_ERR_UNSUPPORTED, "%s: a K slice of %lld groups does not fit in LDS; use more "
                "splits", what, (long long)gmax);
  if (int rc = check_ws(what, ws, ws_bytes, p.ws_bytes)) return rc;
  q4::GemvArgs a{words, scales, x, y, M, N, K};
  hipError_t e = q4::launch_gemv(*d, a, p, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, what);
}

}  // namespace q4

extern "C" {

int q4_gemv(const uint32_t* words, const uint16_t* scales, const uint16_t* x, uint16_t* y,
            int64_t N, int64_t K, void* ws, size_t ws_bytes, q4_stream_t stream) {
  return q4::gemv_common("q4_gemv", words, scales, x, y, 1, N, K, 0, ws, ws_bytes, stream);
}

int q4_gemv_splitk(const uint32_t* words, const uint16_t* scales, const uint16_t* x,
                   uint16_t* y, int64_t N, int64_t K, int64_t splits, void* ws,
                   size_t ws_bytes, q4_stream_t stream) {
  if (splits < 1) return fail(Q4_ERR_SHAPE, "q4_gemv_splitk: splits = %lld: must be >= 1",
                              (long long)splits);
  return q4::gemv_common("q4_gemv_splitk", words, scales, x, y, 1, N, K, splits, ws, ws_bytes,
                     stream);
}

int q4_gemv_batched(const uint32_t* words, const uint16_t* scales, const uint16_t* X,
                    uint16_t* Y, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                    q4_stream_t stream) {
  return q4::gemv_common("q4_gemv_batched", words, scales, X, Y, M, N, K, 0, ws, ws_bytes, stream);
}

}  // extern "C"

extern "C" {

int q4_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t H, q4_stream_t stream) {
  if (!gu || !out) return fail(Q4_ERR_NULL, "q4_silu_mul: NULL pointer");
  if (M < 1 || H < 8 || H % 8)
    return fail(Q4_ERR_SHAPE, "q4_silu_mul: M = %lld, H = %lld: need M >= 1, H %% 8 == 0",
                (long long)M, (long long)H);
  if (M * H >= ((int64_t)1 << 31))
    return fail(Q4_ERR_UNSUPPORTED, "q4_silu_mul: M * H = %lld: too large", (long long)(M * H));
  if (!aligned(gu, 16) || !aligned(out, 16))
    return fail(Q4_ERR_ALIGN, "q4_silu_mul: pointers not 16-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(gu), b0 = reinterpret_cast<uintptr_t>(out);
  if (a0 < b0 + (uintptr_t)(2 * M * H) && b0 < a0 + (uintptr_t)(4 * M * H))
    return fail(Q4_ERR_SHAPE, "q4_silu_mul: out overlaps gu");
  hipError_t e = q4::launch_silu_mul(gu, out, M, H, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_silu_mul");
}

int q4_embed_rows(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                  const int32_t* tokens, int64_t M, uint16_t* out, q4_stream_t stream) {
  if (!words || !scales || !tokens || !out) return fail(Q4_ERR_NULL, "q4_embed_rows: NULL pointer");
  if (int rc = check_shape(N, K)) return fail(rc, "q4_embed_rows: %s", g_error.c_str());
  if (M < 1 || M > 65535) return fail(Q4_ERR_SHAPE, "q4_embed_rows: M = %lld", (long long)M);
  if (!aligned(words, 16) || !aligned(out, 16) || !aligned(scales, 2) || !aligned(tokens, 4))
    return fail(Q4_ERR_ALIGN, "q4_embed_rows: misaligned pointer");
  hipError_t e = q4::launch_embed_rows(words, scales, N, K, tokens, M, out,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_embed_rows");
}

namespace {
bool spans_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}
int check_rows(const char* what, int64_t M, int64_t K) {
  if (M < 1 || K < 8 || K % 8)
    return fail(Q4_ERR_SHAPE, "%s: M = %lld, K = %lld: need M >= 1, K %% 8 == 0", what,
                (long long)M, (long long)K);
  if (M > INT32_MAX || K / 8 > INT32_MAX)
    return fail(Q4_ERR_UNSUPPORTED, "%s: M = %lld, K = %lld: too large", what, (long long)M,
                (long long)K);
  return Q4_OK;
}
}  // namespace

int q4_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M, int64_t K,
               uint16_t* out, q4_stream_t stream) {
  if (!x || !gamma || !out) return fail(Q4_ERR_NULL, "q4_rmsnorm: NULL pointer");
  if (int rc = check_rows("q4_rmsnorm", M, K)) return rc;
  if (!(eps >= 0.f)) return fail(Q4_ERR_SHAPE, "q4_rmsnorm: eps must be >= 0");
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(out, 16))
    return fail(Q4_ERR_ALIGN, "q4_rmsnorm: pointers not 16-byte aligned");
  if (spans_overlap(out, 2 * M * K, x, 2 * M * K) || spans_overlap(out, 2 * M * K, gamma, 2 * K))
    return fail(Q4_ERR_SHAPE, "q4_rmsnorm: out overlaps an input");
  hipError_t e = q4::launch_rmsnorm(nullptr, x, gamma, eps, M, K, nullptr, out,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_rmsnorm");
}

int q4_add_rmsnorm(const uint16_t* delta, const uint16_t* res_in, const uint16_t* gamma, float eps,
                   int64_t M, int64_t K, uint16_t* res_out, uint16_t* out, q4_stream_t stream) {
  if (!delta || !res_in || !gamma || !res_out || !out)
    return fail(Q4_ERR_NULL, "q4_add_rmsnorm: NULL pointer");
  if (int rc = check_rows("q4_add_rmsnorm", M, K)) return rc;
  if (!(eps >= 0.f)) return fail(Q4_ERR_SHAPE, "q4_add_rmsnorm: eps must be >= 0");
  if (!aligned(delta, 16) || !aligned(res_in, 16) || !aligned(gamma, 16) ||
      !aligned(res_out, 16) || !aligned(out, 16))
    return fail(Q4_ERR_ALIGN, "q4_add_rmsnorm: pointers not 16-byte aligned");
  const int64_t rb = 2 * M * K;
  if ((res_out != res_in && spans_overlap(res_out, rb, res_in, rb)) ||
      spans_overlap(res_out, rb, delta, rb) || spans_overlap(res_out, rb, gamma, 2 * K))
    return fail(Q4_ERR_SHAPE, "q4_add_rmsnorm: res_out overlaps an input");
  if (spans_overlap(out, rb, delta, rb) || spans_overlap(out, rb, res_in, rb) ||
      spans_overlap(out, rb, gamma, 2 * K) || spans_overlap(out, rb, res_out, rb))
    return fail(Q4_ERR_SHAPE, "q4_add_rmsnorm: out overlaps another argument");
  hipError_t e = q4::launch_rmsnorm(delta, res_in, gamma, eps, M, K, res_out, out,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_add_rmsnorm");
}

int q4_gemv_norm(const uint32_t* words, const uint16_t* scales, const uint16_t* res_in,
                 const uint16_t* delta, const uint16_t* gamma, float eps, uint16_t* res_out,
                 uint16_t* y, int64_t N, int64_t K, uint32_t flags, q4_stream_t stream) {
  const char* what = "q4_gemv_norm";
  if (!words || !scales || !res_in || !gamma || !y)
    return fail(Q4_ERR_NULL, "%s: NULL pointer (only delta and res_out may be NULL)", what);
  if (flags & ~(Q4_NORM_GLU | Q4_NORM_EXACT))
    return fail(Q4_ERR_SHAPE, "%s: flags = 0x%x: unknown bits", what, flags);
  const bool glu = (flags & Q4_NORM_GLU) != 0, exact = (flags & Q4_NORM_EXACT) != 0;
  if (int rc = check_shape(glu ? 2 * N : N, K)) return fail(rc, "%s: %s", what, g_error.c_str());
  if (!(eps >= 0.f)) return fail(Q4_ERR_SHAPE, "%s: eps must be >= 0", what);
  if (!aligned(words, 16) || !aligned(scales, 2) || !aligned(res_in, 16) || !aligned(gamma, 16) ||
      (delta && !aligned(delta, 16)) || (res_out && !aligned(res_out, 16)) || !aligned(y, 2))
    return fail(Q4_ERR_ALIGN, "%s: misaligned pointer", what);
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  if ((size_t)(K / 32) * (exact ? 192 : 64) > d->lds_per_block)
    return fail(Q4_ERR_UNSUPPORTED, "%s: K = %lld: the %s staging does not fit in LDS", what,
                (long long)K, exact ? "exact" : "factored");
  const int64_t rows = glu ? 2 * N : N, vb = 2 * K;
  const int64_t wb = rows * K / 2, sb = rows * K / 16, yb = 2 * N;
  auto any = [&](const void* p, int64_t pb, std::initializer_list<std::pair<const void*, int64_t>> l) {
    for (auto& q : l)
      if (q.first && spans_overlap(p, pb, q.first, q.second)) return true;
    return false;
  };
  if (any(y, yb, {{words, wb}, {scales, sb}, {res_in, vb}, {delta, vb}, {gamma, vb}, {res_out, vb}}))
    return fail(Q4_ERR_SHAPE, "%s: y overlaps another argument", what);
  if (res_out && any(res_out, vb, {{words, wb}, {scales, sb}, {res_in, vb}, {delta, vb}, {gamma, vb}}))
    return fail(Q4_ERR_SHAPE, "%s: res_out overlaps an input (it must be a buffer of its own)",
                what);
  q4::NormIn nin;
  nin.delta = delta;
  nin.res_in = res_in;
  nin.gamma = gamma;
  nin.res_out = res_out;
  nin.eps = eps;
  nin.exact = exact;
  hipError_t e = q4::launch_gemv_norm_in(*d, words, scales, nin, y, N, K, glu,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, what);
}

int q4_argmax(const uint16_t* x, int64_t M, int64_t N, int32_t* out, q4_stream_t stream) {
  if (!x || !out) return fail(Q4_ERR_NULL, "q4_argmax: NULL pointer");
  if (M < 1 || N < 1 || M > INT32_MAX || N > INT32_MAX)
    return fail(Q4_ERR_SHAPE, "q4_argmax: M = %lld, N = %lld", (long long)M, (long long)N);
  if (!aligned(x, 2) || !aligned(out, 4)) return fail(Q4_ERR_ALIGN, "q4_argmax: misaligned");
  if (spans_overlap(out, 4 * M, x, 2 * M * N))
    return fail(Q4_ERR_SHAPE, "q4_argmax: out overlaps x");
  hipError_t e = q4::launch_argmax(x, M, N, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_argmax");
}

size_t q4_format_weight_bytes(uint32_t format, int64_t N, int64_t K) {
  if (N < 1 || K < 32 || K % 32 || format > Q4_FMT_AF4_G64_F16) return 0;
  if (format >= Q4_FMT_AF4_G64 && K % 64) return 0;
  switch (format) {
    case Q4_FMT_Q3F16_1: return (size_t)N * (size_t)(K / 32) * (12 + 2);
    case Q4_FMT_Q4F32_1: return (size_t)N * (size_t)(K / 32) * (16 + 4);
    case Q4_FMT_AF4_G64:
    case Q4_FMT_AF4_G64_F16: return (size_t)N * (size_t)(K / 64) * (32 + 2 + 2);
    default: return (size_t)N * (size_t)(K / 32) * (16 + 2);
  }
}

int q4_gemv_format(uint32_t format, const uint32_t* words, const void* scales,
                   const uint16_t* biases, const void* x, void* y, int64_t N, int64_t K,
                   q4_stream_t stream) {
  const uint32_t load = format & (Q4_FMT_LOAD_STAGED | Q4_FMT_LOAD_DIRECT);
  format &= ~(Q4_FMT_LOAD_STAGED | Q4_FMT_LOAD_DIRECT);
  if (format < Q4_FMT_Q3F16_1 || format > Q4_FMT_AF4_G64_F16)
    return fail(Q4_ERR_SHAPE, "q4_gemv_format: format = %u: unknown", format);
  if (load && (format != Q4_FMT_Q3F16_1 || load == (Q4_FMT_LOAD_STAGED | Q4_FMT_LOAD_DIRECT)))
    return fail(Q4_ERR_SHAPE, "q4_gemv_format: a load bit is for q3f16_1 only, one at a time");
  if (!words || !scales || !x || !y) return fail(Q4_ERR_NULL, "q4_gemv_format: NULL pointer");
  const bool affine = format == Q4_FMT_AF4_G64 || format == Q4_FMT_AF4_G64_F16;
  const bool f32 = format == Q4_FMT_Q4F32_1;
  if (affine != (biases != nullptr))
    return fail(affine ? Q4_ERR_NULL : Q4_ERR_SHAPE,
                "q4_gemv_format: biases must be given for the affine format only");
  if (N < 1 || N > INT32_MAX || K < 32 || K > 32768 || K % (affine ? 64 : 32))
    return fail(Q4_ERR_SHAPE, "q4_gemv_format: N = %lld, K = %lld", (long long)N, (long long)K);
  const size_t es = f32 ? 4 : 2;
  if (!aligned(words, format == Q4_FMT_Q3F16_1 ? 4 : 16) || !aligned(scales, es) ||
      (biases && !aligned(biases, 2)) || !aligned(x, 16) || !aligned(y, es))
    return fail(Q4_ERR_ALIGN, "q4_gemv_format: misaligned pointer");
  const int64_t wb = N * (K / 32) * (format == Q4_FMT_Q3F16_1 ? 12 : 16);
  const int64_t groups = N * (K / (affine ? 64 : 32));
  const int64_t yb = N * (int64_t)es;
  if (spans_overlap(y, yb, words, wb) || spans_overlap(y, yb, scales, groups * (int64_t)es) ||
      (biases && spans_overlap(y, yb, biases, 2 * groups)) || spans_overlap(y, yb, x, K * (int64_t)es))
    return fail(Q4_ERR_SHAPE, "q4_gemv_format: y overlaps an input");
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "q4_gemv_format: no HIP device");
  const int staged = load == Q4_FMT_LOAD_STAGED ? 1 : load == Q4_FMT_LOAD_DIRECT ? 0 : -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (format == Q4_FMT_Q3F16_1)
    e = q4::launch_gemv_q3(*d, words, static_cast<const uint16_t*>(scales),
                           static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), N, K,
                           staged, st);
  else if (affine)
    e = q4::launch_gemv_affine(*d, words, static_cast<const uint16_t*>(scales), biases,
                               static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), N, K,
                               format == Q4_FMT_AF4_G64, st);
  else
    e = q4::launch_gemv_format(*d, (int)format, words, scales, biases, x, y, N, K, st);
  return e == hipSuccess ? ok() : device_error(e, "q4_gemv_format");
}

int q4_probe_read(const void* buf, size_t bytes, uint32_t* sink, int64_t blocks,
                  q4_stream_t stream) {
  if (!buf || !sink) return fail(Q4_ERR_NULL, "q4_probe_read: NULL pointer");
  if (bytes == 0 || bytes % 16) return fail(Q4_ERR_SHAPE, "q4_probe_read: bytes %% 16 != 0");
  if (!aligned(buf, 16)) return fail(Q4_ERR_ALIGN, "q4_probe_read: buf not 16-byte aligned");
  if (blocks < 0 || blocks > INT32_MAX) return fail(Q4_ERR_SHAPE, "q4_probe_read: bad blocks");
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "q4_probe_read: no HIP device");
  hipError_t e = q4::launch_probe_read(*d, buf, bytes, sink, blocks,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_probe_read");
}

int q4_probe_copy(const void* src, void* dst, size_t bytes, q4_stream_t stream) {
  if (!src || !dst) return fail(Q4_ERR_NULL, "q4_probe_copy: NULL pointer");
  if (bytes == 0 || bytes % 16) return fail(Q4_ERR_SHAPE, "q4_probe_copy: bytes %% 16 != 0");
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(Q4_ERR_ALIGN, "q4_probe_copy: pointers not 16-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(Q4_ERR_SHAPE, "q4_probe_copy: overlap");
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "q4_probe_copy: no HIP device");
  hipError_t e = q4::launch_probe_copy(*d, src, dst, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : device_error(e, "q4_probe_copy");
}

}  // extern "C"
