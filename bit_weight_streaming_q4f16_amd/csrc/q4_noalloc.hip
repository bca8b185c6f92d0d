// q4_gemv_batched_noalloc: q4_gemv_batched for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The split-K partials that q4_gemv_batched keeps in a
// caller workspace live here in one file-scope device array instead; the caller
// still passes inputs and outputs.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken with hipGetSymbolAddress once per device (each GPU
// holds its own copy of the array at its own address) and only that address is
// ever handed to a kernel.
#include <mutex>

#include "q4f16.h"
#include "q4_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[Q4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (taken once per device,
// with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) {
    (void)hipGetLastError();
    return q4::api_fail(Q4_ERR_DEVICE, "q4_gemv_batched_noalloc: hipGetDevice: %s",
                        hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices)
    return q4::api_fail(Q4_ERR_DEVICE, "q4_gemv_batched_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) {
      (void)hipGetLastError();
      return q4::api_fail(Q4_ERR_DEVICE,
                          "q4_gemv_batched_noalloc: hipGetSymbolAddress(scratch): %s",
                          hipGetErrorString(e));
    }
    if (!p)
      return q4::api_fail(Q4_ERR_DEVICE, "q4_gemv_batched_noalloc: scratch has no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return Q4_OK;
}

}  // namespace

extern "C" {

int q4_gemv_batched_noalloc(const uint32_t* words, const uint16_t* scales, const uint16_t* X,
                            uint16_t* Y, int64_t M, int64_t N, int64_t K, q4_stream_t stream) {
  const char* what = "q4_gemv_batched_noalloc";
  if (int rc = q4::gemv_validate(what, words, scales, X, Y, M, N, K)) return rc;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  const size_t need = q4::plan_auto(*d, M, N, K).ws_bytes;
  if (need > (size_t)Q4_NOALLOC_SCRATCH_BYTES)
    return q4::api_fail(Q4_ERR_WORKSPACE,
                        "%s: M = %lld, N = %lld, K = %lld needs %zu bytes of split-K partials; "
                        "the static scratch holds %d (use q4_gemv_batched with a workspace)",
                        what, (long long)M, (long long)N, (long long)K, need,
                        Q4_NOALLOC_SCRATCH_BYTES);
  void* p = nullptr;
  if (int rc = scratch_ptr(&p)) return rc;
  return q4::gemv_common(what, words, scales, X, Y, M, N, K, 0, p,
                         (size_t)Q4_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
