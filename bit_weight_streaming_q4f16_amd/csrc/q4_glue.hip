// Feed-forward glue between the gate/up and down projections (Zero TVM
// documentation, "Decode loop"): out = fp16(silu(gate) * up), as a standalone
// kernel (the persistent decode-step kernel forms the same values while it stages
// the down projection's input).  Eight outputs per thread: one 16-byte load of
// gate, one of up, one 16-byte store.
#include "q4_internal.h"
#include "q4_device.h"

namespace q4 {
namespace {

__global__ __launch_bounds__(kBlock) void k_silu_mul(const uint4* __restrict__ gu,
                                                     uint4* __restrict__ out,
                                                     int blocks_per_row, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= total) return;
  const int64_t m = i / blocks_per_row, b = i % blocks_per_row;
  const uint4 g4 = gu[m * 2 * blocks_per_row + b];
  const uint4 u4 = gu[m * 2 * blocks_per_row + blocks_per_row + b];
  const h8_t g = __builtin_bit_cast(h8_t, g4), u = __builtin_bit_cast(h8_t, u4);
  h8_t h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = silu_mul_h(g[e], u[e]);
  out[m * blocks_per_row + b] = __builtin_bit_cast(uint4, h);
}

}  // namespace

hipError_t launch_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t H,
                           hipStream_t s) {
  const int64_t bpr = H / 8, total = M * bpr;
  const int64_t grid = (total + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)grid), dim3(kBlock), 0, s,
                     reinterpret_cast<const uint4*>(gu), reinterpret_cast<uint4*>(out), (int)bpr,
                     total);
  return hipGetLastError();
}

}  // namespace q4
