// Decode-step plans (include/q4f16.h: q4_step_plan_*, q4_step_run, q4_step_status,
// q4_decode_step).  A list of GEMV descriptors is planned once on the host --
// validation, dependencies, the partition of the rows over the workgroups, the
// launch shape -- into a caller-owned host buffer, and its device tables are
// written into the caller's workspace by small kernels on the caller's stream.
// A run then only launches: the library allocates nothing, frees nothing, keeps
// no state between calls and never waits for the device (q4_step_status, which
// exists to report the persistent kernels' error word, is the one call that
// does).
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "q4f16.h"
#include "q4_internal.h"
#include "q4_step.h"
#include "q4_formats.h"
#include "q4_step_mfma.h"
#include "q4_tok.h"

namespace {

constexpr uint32_t kMagic = 0x51345031u;       // "Q4P1"
constexpr uint32_t kPlanVersion = 1;
constexpr size_t kCtlBytes = (size_t)q4::kCtlWords * 4;

enum Mode : int32_t { kModeStep = 1, kModeStepM = 2, kModeEach = 3 };

// One kernel per descriptor: the descriptor and its GEMV plan.
struct EachEntry {
  q4_layer layer;
  q4::GemvPlan plan;
};

// The plan as it sits in the caller's buffer: this header, then n EachEntry.
struct PlanHeader {
  uint32_t magic, version;
  int32_t device, mode;
  int64_t n, M;
  uint32_t flags, pad;
  const void* ws;              // the workspace the tables were written to
  uint64_t ws_bytes;           // bytes a run needs
  q4::StepLaunch launch;       // modes 1 and 2
  uint64_t glue_off;           // mode 3: workspace offset of the glue output
};

std::vector<q4::StepLayer> to_step_layers(const q4_layer* layers, int64_t n) {
  std::vector<q4::StepLayer> v((size_t)n);
  for (int64_t i = 0; i < n; ++i)
    v[(size_t)i] = q4::StepLayer{layers[i].words, layers[i].scales, layers[i].x, layers[i].y,
                                 layers[i].N, layers[i].K, layers[i].x_op, layers[i].format,
                                 layers[i].biases};
  return v;
}

// Lists in which many descriptors wait for another run faster as one kernel per
// GEMV: in the persistent kernel every waiting GEMV pays its hand-over and its
// arithmetic on the critical path (measured on MI355X: 9.3 us per dependent GEMV
// against about 7 us per launched GEMV), so beyond a quarter of the list waiting
// the launches win, unless the caller asks for the persistent kernel.
bool dependency_bound(int64_t n, int waiting, uint32_t flags) {
  return !(flags & Q4_STEP_PERSISTENT) && 4 * (int64_t)waiting > n;
}

// The chosen way of running a list, with what each way needs.
struct Choice {
  int32_t mode = kModeEach;
  q4::StepLaunch launch{};
  std::vector<uint8_t> table;  // modes 1 and 2: the device tables
  std::vector<q4::GemvPlan> plans;
  size_t glue_off = 0, ws_bytes = 0;
};

Choice choose(const q4::DeviceInfo& d, const q4_layer* layers, int64_t n, int64_t M,
              uint32_t flags) {
  Choice c;
  const bool each = (flags & Q4_STEP_LAUNCH_EACH) != 0;
  const bool ordered = (flags & Q4_STEP_ORDERED) != 0;
  if (!each && M > 1) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n);
    q4::MStepPlan p = q4::plan_step_mfma(d, sl.data(), n, (int)M, ordered);
    int waiting = 0, per_cu = 0;
    for (const q4::MStepDesc& sd : p.desc) waiting += sd.dep >= 0;
    if (p.ok && !dependency_bound(n, waiting, flags) &&
        q4::step_mfma_occupancy(p, &per_cu) == hipSuccess && per_cu >= 1) {
      c.mode = kModeStepM;
      c.launch = q4::step_mfma_launch_of(p);
      q4::step_mfma_table_bytes(p, &c.table);
      c.ws_bytes = c.launch.ws_bytes;
      return c;
    }
    (void)hipGetLastError();
  }
  // a single GEMV at M = 1 is faster as one GEMV kernel (262144 x 3072: 73.7
  // against 80.7 us; qkv-sized: 8.7 against ~14 us), unless the caller asks
  // for the persistent kernel
  if (!each && M == 1 && (n > 1 || (flags & Q4_STEP_PERSISTENT))) {
    std::vector<q4::StepLayer> sl = to_step_layers(layers, n);
    q4::StepPlan p = q4::plan_step(d, sl.data(), n, ordered);
    int waiting = 0, per_cu = 0;
    for (const q4::StepDesc& sd : p.desc) waiting += sd.dep >= 0;
    if (p.ok && !dependency_bound(n, waiting, flags) &&
        q4::step_occupancy(p, &per_cu) == hipSuccess && per_cu >= 1) {
      c.mode = kModeStep;
      c.launch = q4::step_launch_of(p);
      q4::step_table_bytes(p, &c.table);
      c.ws_bytes = c.launch.ws_bytes;
      return c;
    }
    (void)hipGetLastError();
  }
  // one kernel per descriptor: the control block, the largest split-K partials of
  // any descriptor, then (for descriptors with Q4_X_SILU_MUL) the largest glue
  // output, M * K fp16
  c.mode = kModeEach;
  c.plans.resize((size_t)n);
  size_t part = 0, glue = 0;
  for (int64_t i = 0; i < n; ++i) {
    // (q3f16_1 and affine layers run as one GEMV kernel, with no split-K partials)
    if (!layers[i].format) c.plans[(size_t)i] = q4::plan_auto(d, M, layers[i].N, layers[i].K);
    part = std::max(part, c.plans[(size_t)i].ws_bytes);
    if (layers[i].x_op) glue = std::max(glue, (size_t)(2 * M * layers[i].K));
  }
  c.glue_off = (kCtlBytes + part + 255) & ~(size_t)255;
  c.ws_bytes = c.glue_off + glue;
  return c;
}

constexpr uint32_t kFlags = Q4_STEP_LAUNCH_EACH | Q4_STEP_ORDERED | Q4_STEP_PERSISTENT;

// Every argument check, before anything is enqueued.
int validate(const char* what, const q4_layer* layers, int64_t n, int64_t M, uint32_t flags) {
  if (!layers) return q4::api_fail(Q4_ERR_NULL, "%s: layers is NULL", what);
  if (n < 1) return q4::api_fail(Q4_ERR_SHAPE, "%s: n_layers = %lld: must be >= 1", what,
                                 (long long)n);
  if (n > (1 << 20))
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: n_layers = %lld: too many", what, (long long)n);
  if (M < 1 || M > q4::kMaxM)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: M = %lld: must be in [1, %d]", what, (long long)M,
                        q4::kMaxM);
  if (flags & ~kFlags) return q4::api_fail(Q4_ERR_SHAPE, "%s: unknown flags 0x%x", what, flags);
  char w[96];
  for (int64_t i = 0; i < n; ++i) {
    const q4_layer& L = layers[i];
    snprintf(w, sizeof w, "%s: layers[%lld]", what, (long long)i);
    if (L.x_op > Q4_X_SILU_MUL)
      return q4::api_fail(Q4_ERR_SHAPE, "%s: x_op = %u: unknown", w, L.x_op);
    const bool aff = L.format == Q4_FMT_AF4_G64 || L.format == Q4_FMT_AF4_G64_F16;
    if (L.format != 0 && L.format != Q4_FMT_Q3F16_1 && !aff)
      return q4::api_fail(Q4_ERR_SHAPE, "%s: format = %u: must be 0 (q4f16_1), "
                          "Q4_FMT_Q3F16_1, Q4_FMT_AF4_G64 or Q4_FMT_AF4_G64_F16", w, L.format);
    if (L.format && M != 1)
      return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: format %u layers run at M = 1 only", w,
                          L.format);
    if (L.format && L.K > 32768)
      return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: format %u layers take K <= 32768", w,
                          L.format);
    if (aff != (L.biases != nullptr))
      return q4::api_fail(aff ? Q4_ERR_NULL : Q4_ERR_SHAPE,
                          "%s: biases must be given for the affine formats only", w);
    if (aff && L.K % 64)
      return q4::api_fail(Q4_ERR_SHAPE, "%s: K = %lld: the affine formats take K %% 64 == 0", w,
                          (long long)L.K);
    if (int rc = q4::gemv_validate(w, L.words, L.scales, L.x, L.y, M, L.N, L.K,
                                   L.x_op ? 2 * L.K : L.K, L.format, L.biases))
      return rc;
  }
  return Q4_OK;
}

size_t plan_bytes_for(int64_t n) { return sizeof(PlanHeader) + (size_t)n * sizeof(EachEntry); }

int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess) {
    (void)hipGetLastError();
    return Q4_ERR_DEVICE;
  }
  return Q4_OK;
}

// Plan into `plan` and enqueue the set-up writes into ws (see q4_step_plan_init).
int plan_init(const char* what, const q4_layer* layers, int64_t n, int64_t M, uint32_t flags,
              void* plan, size_t plan_bytes, void* ws, size_t ws_bytes, hipStream_t s) {
  if (int rc = validate(what, layers, n, M, flags)) return rc;
  if (!plan) return q4::api_fail(Q4_ERR_NULL, "%s: plan is NULL", what);
  if (plan_bytes < plan_bytes_for(n))
    return q4::api_fail(Q4_ERR_WORKSPACE, "%s: the plan needs %zu bytes, got %zu", what,
                        plan_bytes_for(n), plan_bytes);
  if (reinterpret_cast<uintptr_t>(plan) % 8)
    return q4::api_fail(Q4_ERR_ALIGN, "%s: plan not 8-byte aligned", what);
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  Choice c = choose(*d, layers, n, M, flags);
  if (int rc = q4::ws_validate(what, ws, ws_bytes, c.ws_bytes)) return rc;
  hipError_t e = hipSuccess;
  if (c.mode == kModeStep || c.mode == kModeStepM) {
    e = c.mode == kModeStep ? q4::step_prepare(c.launch) : q4::step_mfma_prepare(c.launch);
    if (e == hipSuccess) e = q4::zero_words(ws, c.launch.clear_bytes / 4, s);
    if (e == hipSuccess)
      e = q4::write_table(static_cast<uint8_t*>(ws) + c.launch.table_off, c.table.data(),
                          c.table.size(), s);
  } else {
    e = q4::zero_words(ws, q4::kCtlWords, s);
  }
  if (e != hipSuccess) return q4::device_fail(e, what);
  PlanHeader h{};
  h.magic = kMagic;
  h.version = kPlanVersion;
  h.device = d->id;
  h.mode = c.mode;
  h.n = n;
  h.M = M;
  h.flags = flags;
  h.ws = ws;
  h.ws_bytes = c.ws_bytes;
  h.launch = c.launch;
  h.glue_off = c.glue_off;
  memcpy(plan, &h, sizeof h);
  EachEntry* ent = reinterpret_cast<EachEntry*>(static_cast<uint8_t*>(plan) + sizeof h);
  for (int64_t i = 0; i < n; ++i) {
    EachEntry en{};
    en.layer = layers[i];
    if (c.mode == kModeEach) en.plan = c.plans[(size_t)i];
    memcpy(ent + i, &en, sizeof en);
  }
  return q4::api_ok();
}

int run(const char* what, const void* plan, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!plan) return q4::api_fail(Q4_ERR_NULL, "%s: plan is NULL", what);
  PlanHeader h;
  memcpy(&h, plan, sizeof h);
  if (h.magic != kMagic || h.version != kPlanVersion)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: not a plan made by q4_step_plan_init", what);
  if (ws != h.ws)
    return q4::api_fail(Q4_ERR_WORKSPACE, "%s: ws %p is not the workspace the plan was made "
                        "with (%p)", what, ws, h.ws);
  if (int rc = q4::ws_validate(what, ws, ws_bytes, h.ws_bytes)) return rc;
  int dev = -1;
  if (current_device(&dev) || dev != h.device)
    return q4::api_fail(Q4_ERR_DEVICE, "%s: the plan is for device %d, the current one is %d",
                        what, h.device, dev);
  hipError_t e = hipSuccess;
  if (h.mode == kModeStep) {
    e = q4::launch_step(h.launch, ws, s);
  } else if (h.mode == kModeStepM) {
    e = q4::launch_step_mfma(h.launch, ws, s);
  } else {
    const q4::DeviceInfo* d = q4::device_info();
    if (!d) return q4::api_fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* glue = reinterpret_cast<uint16_t*>(base + h.glue_off);
    const EachEntry* ent =
        reinterpret_cast<const EachEntry*>(static_cast<const uint8_t*>(plan) + sizeof h);
    for (int64_t i = 0; i < h.n && e == hipSuccess; ++i) {
      EachEntry en;
      memcpy(&en, ent + i, sizeof en);
      const q4_layer& L = en.layer;
      const uint16_t* x = L.x;
      if (L.x_op == Q4_X_SILU_MUL) {
        e = q4::launch_silu_mul(L.x, glue, h.M, L.K, s);
        x = glue;
      }
      if (e == hipSuccess && L.format == Q4_FMT_Q3F16_1) {
        e = q4::launch_gemv_q3(*d, L.words, L.scales, x, L.y, L.N, L.K, -1, s);
        continue;
      }
      if (e == hipSuccess && (L.format == Q4_FMT_AF4_G64 || L.format == Q4_FMT_AF4_G64_F16)) {
        e = q4::launch_gemv_affine(*d, L.words, L.scales, L.biases, x, L.y, L.N, L.K,
                                   L.format == Q4_FMT_AF4_G64, s);
        continue;
      }
      const q4::GemvArgs a{L.words, L.scales, x, L.y, h.M, L.N, L.K};
      if (e == hipSuccess) e = q4::launch_gemv(*d, a, en.plan, base + kCtlBytes, s);
    }
  }
  return e == hipSuccess ? q4::api_ok() : q4::device_fail(e, what);
}

const char* wait_name(unsigned code) {
  switch (code) {
    case q4::kErrLocal: return "a sync wave's wait for its workgroup's compute waves";
    case q4::kErrCounter: return "a wait for another GEMV's completion counter";
    case q4::kErrX: return "a compute wave's wait for its GEMV's staged input";
    case q4::kErrTag: return "a wait for values handed over by the producing GEMV";
    case q4::kErrRegion: return "a wait for an LDS region's previous GEMV";
    default: return "an unknown wait";
  }
}

}  // namespace

extern "C" {

size_t q4_step_plan_bytes(int64_t n_layers) {
  if (n_layers < 1 || n_layers > (1 << 20)) return 0;
  return plan_bytes_for(n_layers);
}

size_t q4_decode_step_workspace_bytes(const q4_layer* layers, int64_t n_layers, int64_t M,
                                      uint32_t flags) {
  if (!layers || n_layers < 1 || n_layers > (1 << 20) || M < 1 || M > q4::kMaxM ||
      (flags & ~kFlags))
    return 0;
  for (int64_t i = 0; i < n_layers; ++i)
    if (layers[i].N < 1 || layers[i].K < 32 || layers[i].K % 32) return 0;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return 0;
  return choose(*d, layers, n_layers, M, flags).ws_bytes;
}

int q4_step_plan_init(const q4_layer* layers, int64_t n_layers, int64_t M, uint32_t flags,
                      void* plan, size_t plan_bytes, void* ws, size_t ws_bytes,
                      q4_stream_t stream) {
  return plan_init("q4_step_plan_init", layers, n_layers, M, flags, plan, plan_bytes, ws,
                   ws_bytes, static_cast<hipStream_t>(stream));
}

int q4_step_run(const void* plan, void* ws, size_t ws_bytes, q4_stream_t stream) {
  return run("q4_step_run", plan, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int q4_step_status(void* ws, q4_stream_t stream) {
  if (!ws) return q4::api_fail(Q4_ERR_NULL, "q4_step_status: ws is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, ws, sizeof word, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return q4::device_fail(e, "q4_step_status");
  if (!word) return q4::api_ok();
  // clear it for the next check (a kernel, as every write the library enqueues)
  e = q4::zero_words(ws, 1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return q4::device_fail(e, "q4_step_status");
  const unsigned code = word & 0x7Fu, gemv = (word >> 8);
  if (word & q4::kErrTokenKernel)
    return q4::api_fail(Q4_ERR_TIMEOUT,
                        "q4_step_status: %s ran out in the whole-token kernel (error word "
                        "0x%08x: code %u, stage %d of the step); the tokens and logits of that "
                        "run are not valid", wait_name(code), word, code, (int)gemv - 1);
  return q4::api_fail(Q4_ERR_TIMEOUT,
                      "q4_step_status: %s ran out (error word 0x%08x: code %u, layers[%d]); "
                      "the outputs of that step are not valid", wait_name(code), word, code,
                      (int)gemv - 1);
}

int q4_decode_step_flags(const q4_layer* layers, int64_t n_layers, int64_t M, uint32_t flags,
                         void* ws, size_t ws_bytes, q4_stream_t stream) {
  const char* what = "q4_decode_step";
  if (n_layers < 1 || n_layers > (1 << 20))
    return validate(what, layers, n_layers, M, flags);
  std::vector<uint64_t> plan((plan_bytes_for(n_layers) + 7) / 8);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (int rc = plan_init(what, layers, n_layers, M, flags, plan.data(), plan.size() * 8, ws,
                         ws_bytes, s))
    return rc;
  return run(what, plan.data(), ws, ws_bytes, s);
}

int q4_decode_step(const q4_layer* layers, int64_t n_layers, int64_t M, void* ws,
                   size_t ws_bytes, q4_stream_t stream) {
  return q4_decode_step_flags(layers, n_layers, M, 0, ws, ws_bytes, stream);
}

}  // extern "C"
