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
               int64_t x_cols) {
  if (!words) return fail(Q4_ERR_NULL, "%s: words is NULL", what);
  if (!scales) return fail(Q4_ERR_NULL, "%s: scales is NULL", what);
  if (!x) return fail(Q4_ERR_NULL, "%s: x is NULL", what);
  if (!y) return fail(Q4_ERR_NULL, "%s: y is NULL", what);
  if (M < 1 || M > q4::kMaxM)
    return fail(Q4_ERR_SHAPE, "%s: M = %lld: must be in [1, %d]", what, (long long)M, q4::kMaxM);
  int rc = check_shape(N, K);
  if (rc) return fail(rc, "%s: %s", what, g_error.c_str());
  if (!aligned(words, 16)) return fail(Q4_ERR_ALIGN, "%s: words %p not 16-byte aligned", what,
                                       (const void*)words);
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
  if (overlaps(words, N * K / 2) || overlaps(scales, N * K / 16) || overlaps(x, 2 * M * x_cols))
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
    default: return "Q4_ERR_UNKNOWN";
  }
}

const char* q4_last_error(void) { return g_error.c_str(); }

int q4_version(void) { return 100; }

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
                  const uint16_t* x, const uint16_t* y, int64_t M, int64_t N, int64_t K) {
  return check_gemv(what, words, scales, x, y, M, N, K, K);
}

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

namespace {

// Device copies of step descriptor tables, keyed by their contents (pointers,
// shapes, dependencies) and device.  A table is uploaded on first use of a
// layer list and reused by every later call with the same list; the least
// recently used of kMaxTables entries is freed when a new one is needed.
struct TableEntry {
  int dev = -1;
  std::vector<uint8_t> bytes;
  void* dptr = nullptr;
  uint64_t last_use = 0;
};
constexpr size_t kMaxTables = 16;
std::mutex g_table_mutex;
std::vector<TableEntry> g_tables;
uint64_t g_table_clock = 0;

const void* device_table(const void* host, size_t bytes, int dev, hipStream_t s, hipError_t* err) {
  std::lock_guard<std::mutex> lock(g_table_mutex);
  for (TableEntry& e : g_tables) {
    if (e.dev == dev && e.bytes.size() == bytes && memcmp(e.bytes.data(), host, bytes) == 0) {
      e.last_use = ++g_table_clock;
      return e.dptr;
    }
  }
  if (g_tables.size() >= kMaxTables) {
    size_t lru = 0;
    for (size_t i = 1; i < g_tables.size(); ++i)
      if (g_tables[i].last_use < g_tables[lru].last_use) lru = i;
    (void)hipFree(g_tables[lru].dptr);      // synchronises: no launch still reads it
    g_tables.erase(g_tables.begin() + (ptrdiff_t)lru);
  }
  TableEntry e;
  e.dev = dev;
  e.bytes.assign(static_cast<const uint8_t*>(host), static_cast<const uint8_t*>(host) + bytes);
  if ((*err = hipMalloc(&e.dptr, bytes)) != hipSuccess) return nullptr;
  if ((*err = hipMemcpyAsync(e.dptr, e.bytes.data(), bytes, hipMemcpyHostToDevice, s)) !=
      hipSuccess) {
    (void)hipFree(e.dptr);
    return nullptr;
  }
  e.last_use = ++g_table_clock;
  g_tables.push_back(std::move(e));
  return g_tables.back().dptr;
}

std::vector<q4::StepLayer> to_step_layers(const q4_layer* layers, int64_t n) {
  std::vector<q4::StepLayer> v((size_t)n);
  for (int64_t i = 0; i < n; ++i)
    v[(size_t)i] = q4::StepLayer{layers[i].words, layers[i].scales, layers[i].x, layers[i].y,
                                 layers[i].N, layers[i].K, layers[i].x_op};
  return v;
}

// The persistent path applies to M == 1 lists whose rows fit its item shape,
// when one workgroup of the step kernel fits on every compute unit.
// Lists in which many descriptors wait for another run faster as one kernel per
// GEMV: in the persistent kernel every waiting GEMV pays its hand-over and its
// arithmetic on the critical path (measured on MI355X: 9.3 us per dependent GEMV
// against about 7 us per launched GEMV), so beyond a quarter of the list waiting the
// launches win, unless the caller asks for the persistent kernel.
bool dependency_bound(int64_t n, int waiting, uint32_t flags) {
  return !(flags & Q4_STEP_PERSISTENT) && 4 * (int64_t)waiting > n;
}

bool use_persistent(const q4::DeviceInfo& d, const q4::StepPlan& p, int64_t M, uint32_t flags) {
  if (M != 1 || (flags & Q4_STEP_LAUNCH_EACH) || !p.ok) return false;
  // a single GEMV is faster as one GEMV kernel (262144 x 3072: 73.7 against 80.7 us;
  // qkv-sized: 8.7 against ~14 us), unless the caller asks for the persistent kernel
  if (p.desc.size() == 1 && !(flags & Q4_STEP_PERSISTENT)) return false;
  int waiting = 0;
  for (const q4::StepDesc& sd : p.desc) waiting += sd.dep >= 0;
  if (dependency_bound((int64_t)p.desc.size(), waiting, flags)) return false;
  int per_cu = 0;
  if (q4::step_occupancy(p, &per_cu) != hipSuccess || per_cu < 1) {
    (void)hipGetLastError();
    return false;
  }
  (void)d;
  return true;
}

// One kernel per descriptor: the largest split-K partials of any descriptor, then
// (for descriptors with Q4_X_SILU_MUL) the largest glue output, M * K fp16.
struct EachLayout {
  std::vector<q4::GemvPlan> plans;
  size_t glue_off = 0, bytes = 0;
};
EachLayout each_layout(const q4::DeviceInfo& d, const q4_layer* layers, int64_t n, int64_t M) {
  EachLayout e;
  e.plans.resize((size_t)n);
  size_t part = 0, glue = 0;
  for (int64_t i = 0; i < n; ++i) {
    e.plans[(size_t)i] = q4::plan_auto(d, M, layers[i].N, layers[i].K);
    part = std::max(part, e.plans[(size_t)i].ws_bytes);
    if (layers[i].x_op) glue = std::max(glue, (size_t)(2 * M * layers[i].K));
  }
  e.glue_off = (part + 255) & ~(size_t)255;
  e.bytes = glue ? e.glue_off + glue : part;
  return e;
}

bool any_x_op(const q4_layer* layers, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (layers[i].x_op) return true;
  return false;
}

}  // namespace

extern "C" {

size_t q4_decode_step_workspace_bytes(const q4_layer* layers, int64_t n_layers, int64_t M,
                                      uint32_t flags) {
  if (!layers || n_layers < 1 || M < 1 || M > q4::kMaxM) return 0;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return 0;
  for (int64_t i = 0; i < n_layers; ++i) {
    const q4_layer& L = layers[i];
    if (L.N < 1 || L.K < 32 || L.K % 32) return 0;
  }
  size_t need = each_layout(*d, layers, n_layers, M).bytes;
  if (M > 1 && !(flags & Q4_STEP_LAUNCH_EACH)) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n_layers);
    q4::MStepPlan p = q4::plan_step_mfma(*d, sl.data(), n_layers, (int)M,
                                         (flags & Q4_STEP_ORDERED) != 0);
    if (p.ok) need = std::max(need, q4::step_mfma_workspace_bytes(p));
  }
  if (M == 1 && !(flags & Q4_STEP_LAUNCH_EACH)) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n_layers);
    q4::StepPlan p = q4::plan_step(*d, sl.data(), n_layers, (flags & Q4_STEP_ORDERED) != 0);
    size_t b = q4::step_workspace_bytes(p);
    if (b > need) need = b;
  }
  return need;
}

int q4_decode_step(const q4_layer* layers, int64_t n_layers, int64_t M, uint32_t flags,
                   void* ws, size_t ws_bytes, q4_stream_t stream) {
  if (!layers) return fail(Q4_ERR_NULL, "q4_decode_step: layers is NULL");
  if (n_layers < 1) return fail(Q4_ERR_SHAPE, "q4_decode_step: n_layers = %lld: must be >= 1",
                                (long long)n_layers);
  if (n_layers > (1 << 20))
    return fail(Q4_ERR_UNSUPPORTED, "q4_decode_step: n_layers = %lld: too many",
                (long long)n_layers);
  if (flags & ~(Q4_STEP_LAUNCH_EACH | Q4_STEP_ORDERED | Q4_STEP_WS_CLEAN | Q4_STEP_PERSISTENT))
    return fail(Q4_ERR_SHAPE, "q4_decode_step: unknown flags 0x%x", flags);
  char what[64];
  for (int64_t i = 0; i < n_layers; ++i) {
    const q4_layer& L = layers[i];
    snprintf(what, sizeof what, "q4_decode_step: layers[%lld]", (long long)i);
    if (L.x_op > Q4_X_SILU_MUL)
      return fail(Q4_ERR_SHAPE, "%s: x_op = %u: unknown", what, L.x_op);
    if (L.reserved) return fail(Q4_ERR_SHAPE, "%s: reserved = %u: must be 0", what, L.reserved);
    if (int rc = check_gemv(what, L.words, L.scales, L.x, L.y, M, L.N, L.K,
                            L.x_op ? 2 * L.K : L.K))
      return rc;
  }
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return fail(Q4_ERR_DEVICE, "q4_decode_step: no HIP device");
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (M > 1 && !(flags & Q4_STEP_LAUNCH_EACH)) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n_layers);
    q4::MStepPlan p = q4::plan_step_mfma(*d, sl.data(), n_layers, (int)M,
                                         (flags & Q4_STEP_ORDERED) != 0);
    int per_cu = 0;
    int waiting = 0;
    for (const q4::MStepDesc& sd : p.desc) waiting += sd.dep >= 0;
    if (p.ok && !dependency_bound(n_layers, waiting, flags) &&
        q4::step_mfma_occupancy(p, &per_cu) == hipSuccess && per_cu >= 1) {
      if (int rc = check_ws("q4_decode_step", ws, ws_bytes, q4::step_mfma_workspace_bytes(p)))
        return rc;
      hipError_t e = hipSuccess;
      const size_t db = p.desc.size() * sizeof(q4::MStepDesc);
      std::vector<uint8_t> host(db + p.ranges.size() * sizeof(int));
      std::memcpy(host.data(), p.desc.data(), db);
      if (!p.ranges.empty())
        std::memcpy(host.data() + db, p.ranges.data(), p.ranges.size() * sizeof(int));
      const void* table = device_table(host.data(), host.size(), d->id, s, &e);
      if (!table) return device_error(e, "q4_decode_step: descriptor table");
      const int4* ranges = reinterpret_cast<const int4*>(static_cast<const uint8_t*>(table) + db);
      e = q4::launch_step_mfma(p, static_cast<const q4::MStepDesc*>(table), ranges, ws,
                               (flags & Q4_STEP_WS_CLEAN) != 0, s);
      return e == hipSuccess ? ok() : device_error(e, "q4_decode_step");
    }
    (void)hipGetLastError();
  }
  if (M == 1 && !(flags & Q4_STEP_LAUNCH_EACH)) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n_layers);
    q4::StepPlan p = q4::plan_step(*d, sl.data(), n_layers, (flags & Q4_STEP_ORDERED) != 0);
    if (use_persistent(*d, p, M, flags)) {
      if (int rc = check_ws("q4_decode_step", ws, ws_bytes, q4::step_workspace_bytes(p)))
        return rc;
      hipError_t e = hipSuccess;
      // descriptors, then (range mode) the per-workgroup ranges
      const size_t db = p.desc.size() * sizeof(q4::StepDesc);
      std::vector<uint8_t> host(db + p.ranges.size() * sizeof(int));
      std::memcpy(host.data(), p.desc.data(), db);
      if (!p.ranges.empty())
        std::memcpy(host.data() + db, p.ranges.data(), p.ranges.size() * sizeof(int));
      const void* table = device_table(host.data(), host.size(), d->id, s, &e);
      if (!table) return device_error(e, "q4_decode_step: descriptor table");
      const int4* ranges = reinterpret_cast<const int4*>(static_cast<const uint8_t*>(table) + db);
      e = q4::launch_step(p, static_cast<const q4::StepDesc*>(table), ranges, ws,
                          (flags & Q4_STEP_WS_CLEAN) != 0, s);
      return e == hipSuccess ? ok() : device_error(e, "q4_decode_step");
    }
  }

  const EachLayout el = each_layout(*d, layers, n_layers, M);
  if (int rc = check_ws("q4_decode_step", ws, ws_bytes, el.bytes)) return rc;
  uint16_t* glue = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + el.glue_off);
  for (int64_t i = 0; i < n_layers; ++i) {
    const q4_layer& L = layers[i];
    hipError_t e = hipSuccess;
    const uint16_t* x = L.x;
    if (L.x_op == Q4_X_SILU_MUL) {
      e = q4::launch_silu_mul(L.x, glue, M, L.K, s);
      x = glue;
    }
    q4::GemvArgs a{L.words, L.scales, x, L.y, M, L.N, L.K};
    if (e == hipSuccess) e = q4::launch_gemv(*d, a, el.plans[(size_t)i], ws, s);
    if (e != hipSuccess) {
      snprintf(what, sizeof what, "q4_decode_step: layers[%lld]", (long long)i);
      return device_error(e, what);
    }
  }
  return ok();
}

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
