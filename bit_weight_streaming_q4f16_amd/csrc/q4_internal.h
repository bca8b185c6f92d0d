// Internal interface between the C-ABI layer (q4_api.cpp) and the HIP kernels.
// Not installed; the public interface is include/q4f16.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit load with the non-temporal hint (streamed data that is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr int kBlock = 256;          // threads per workgroup (four wave64s)
constexpr int kMaxSplits = 64;       // split-K slices accepted by q4_gemv_splitk
constexpr int kMaxM = 8;             // rows of the batched (small-M) GEMV

struct DeviceInfo {
  int id = -1;
  int cus = 0;                       // compute units
  size_t lds_per_block = 0;          // bytes of LDS one workgroup may allocate
};

// Properties of the current device (cached per device); nullptr if no device.
const DeviceInfo* device_info();

// The entry points' error reporting (q4_api.cpp): set the calling thread's error
// text and return the status.
int api_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int api_ok();

// The argument checks of one GEMV (null pointers, shape, alignment, overlap); x_cols:
// elements per row of x (0: K); format: 0 (q4f16_1) or Q4_FMT_Q3F16_1 (the words'
// alignment and size).
int gemv_validate(const char* what, const uint32_t* words, const uint16_t* scales,
                  const uint16_t* x, const uint16_t* y, int64_t M, int64_t N, int64_t K,
                  int64_t x_cols = 0, uint32_t format = 0,
                  const uint16_t* biases = nullptr);
// The workspace check (NULL, size, 16-byte alignment) when `need` bytes are needed.
int ws_validate(const char* what, void* ws, size_t have, size_t need);
// Q4_ERR_DEVICE with the HIP error's text.
int device_fail(hipError_t e, const char* what);
// The body of q4_gemv / q4_gemv_batched / q4_gemv_splitk (q4_api.cpp): validate the
// arguments, plan (splits == 0: automatic), check the workspace, launch.
int gemv_common(const char* what, const uint32_t* words, const uint16_t* scales,
                const uint16_t* x, uint16_t* y, int64_t M, int64_t N, int64_t K,
                int64_t splits, void* ws, size_t ws_bytes, void* stream);

// One GEMV as the kernels see it.
struct GemvArgs {
  const uint32_t* words;             // [N][K/8]
  const uint16_t* scales;            // [N][K/32]
  const uint16_t* x;                 // [M][K]
  uint16_t* y;                       // [M][N]
  int64_t M, N, K;
};

// Launch plan of one GEMV: how many K slices and which kernel shape.
struct GemvPlan {
  int splits = 1;                    // K slices (1 = single pass, no workspace)
  int lanes_per_row = 32;            // M <= kMxMax kernels: lanes cooperating on a row
  size_t ws_bytes = 0;               // fp32 partials when splits > 1
};

// Input rows up to which a GEMV runs on the vector units (k_gemv_m1, k_gemv_mx);
// more take the MFMA kernel (at four rows the vector path's LDS reads of X made
// the 151936 x 2048 GEMV 49 -> 64 us).
constexpr int64_t kMxMax = 3;

// Largest number of groups one workgroup stages in LDS for M input rows.
int64_t max_groups_per_slice(const DeviceInfo& d, int64_t M);

// Automatic plan for a shape (used by q4_gemv, q4_gemv_batched, q4_decode_step).
GemvPlan plan_auto(const DeviceInfo& d, int64_t M, int64_t N, int64_t K);
// Plan with an explicit number of slices (q4_gemv_splitk).
GemvPlan plan_splits(const DeviceInfo& d, int64_t M, int64_t N, int64_t K, int splits);

// Enqueue one GEMV with a plan.  ws must hold plan.ws_bytes.  Returns a hipError_t.
hipError_t launch_gemv(const DeviceInfo& d, const GemvArgs& a, const GemvPlan& p, void* ws,
                       hipStream_t s);

hipError_t launch_pack(const uint8_t* codes, uint32_t* words, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_unpack(const uint32_t* words, uint8_t* codes, int64_t N, int64_t K,
                         hipStream_t s);

// The feed-forward glue of the decode loop (Zero TVM documentation, "Decode
// loop"): fp16(silu(g) * u) with silu(g) = g / (1 + exp(-g)), in fp32, rounded to
// nearest even; silu(+inf) = +inf, silu(-inf) = -0 (its limits).
// The product is rounded to fp32 and then to fp16, as written: the empty asm keeps
// the compiler from fusing the two into one mixed-precision instruction (which
// rounds once), so every kernel that forms the glue gets the same bits.
__device__ __forceinline__ _Float16 silu_mul_h(_Float16 g, _Float16 u) {
  const float gf = (float)g;
  float sg;
  if (__builtin_isinf(gf))
    sg = gf > 0.f ? gf : -0.f;
  else
    sg = gf / (1.f + __expf(-gf));
  float p = sg * (float)u;
  asm volatile("" : "+v"(p));
  return (_Float16)p;
}

// RMSNorm of a row of K values (Zero TVM documentation, "Decode loop"), in the
// pieces every kernel that forms it shares, so that they all get the same bits:
// a 256-thread workgroup in which thread t takes the blocks of 8 values t, t + 256,
// ... and sums their squares with fmaf in index order; block_sum adds the 256
// partial sums (a butterfly within each wave, then the four waves in order);
// rms_scale is 1 / sqrt(sum / K + eps); norm_h rounds v * r * gamma to fp32 and
// then to fp16 (the empty asm keeps the compiler from fusing the product and the
// conversion into one mixed-precision instruction, which would round once).
// REUSE: a barrier after the read, so that `red` may be written again.
template <bool REUSE = true>
__device__ __forceinline__ float block_sum(float v, float* red) {   // red: 4 floats
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float t = red[0] + red[1] + red[2] + red[3];
  if (REUSE) __syncthreads();
  return t;
}
__device__ __forceinline__ float rms_scale(float sum_sq, int K, float eps) {
  return 1.f / __builtin_sqrtf(sum_sq / (float)K + eps);
}
__device__ __forceinline__ _Float16 norm_h(_Float16 v, float r, _Float16 g) {
  float p = (float)v * r * (float)g;
  asm volatile("" : "+v"(p));
  return (_Float16)p;
}

// out[m][i] = silu_mul_h(gu[m][i], gu[m][H + i]); H % 8 == 0, 16-byte aligned.
hipError_t launch_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t H,
                           hipStream_t s);

// The operations around the GEMVs (q4_ops.hip).  delta == nullptr: plain RMSNorm.
// A multi-step decode keeps its tokens on the device: with `counter` (M == 1), the
// embedding row is that of seq[counter[0]] instead of tokens[0], and the argmax,
// besides out[0], writes seq[counter[0] + 1] and advances counter[0].
hipError_t launch_embed_rows(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                             const int32_t* tokens, int64_t M, uint16_t* out, hipStream_t s,
                             const int32_t* seq = nullptr, const int32_t* counter = nullptr);
hipError_t launch_rmsnorm(const uint16_t* delta, const uint16_t* res_in, const uint16_t* gamma,
                          float eps, int64_t M, int64_t K, uint16_t* res_out, uint16_t* out,
                          hipStream_t s);
hipError_t launch_argmax(const uint16_t* x, int64_t M, int64_t N, int32_t* out, hipStream_t s,
                         int32_t* seq = nullptr, int32_t* counter = nullptr);
// counter[0] = 0 (a kernel, so that a captured graph holds no memset node).
hipError_t launch_counter_reset(int32_t* counter, hipStream_t s);

// GEMV of a format variant at M = 1 (q4_formats.hip): format 1 q3f16_1, 2 q4f32_1,
// 3 af4g64 (see include/q4f16.h); K <= 32768.
hipError_t launch_gemv_format(const DeviceInfo& d, int format, const uint32_t* W, const void* S,
                              const uint16_t* B, const void* X, void* Y, int64_t N, int64_t K,
                              hipStream_t s);

hipError_t launch_probe_read(const DeviceInfo& d, const void* buf, size_t bytes, uint32_t* sink,
                             int64_t blocks, hipStream_t s);
hipError_t launch_probe_copy(const DeviceInfo& d, const void* src, void* dst, size_t bytes,
                             hipStream_t s);

}  // namespace q4
