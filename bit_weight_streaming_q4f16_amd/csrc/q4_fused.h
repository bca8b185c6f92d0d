// The feed-forward glue of the decode loop (Zero TVM documentation, "Decode
// loop") folded into the gate/up GEMV, so that a decode step launches one kernel
// fewer per block: on this GPU every kernel boundary costs a few microseconds
// whatever the kernel does.  One team computes row i of gate and row i of up
// (rows i and F + i of the gate_up matrix) and writes silu_mul_h(fp16(gate),
// fp16(up)) -- bitwise what the GEMV followed by the glue kernel writes.
#pragma once

#include "q4_internal.h"

namespace q4 {

// The residual add and RMSNorm feeding a GEMV (RMSNorm as the Zero TVM
// documentation's decode loop places it), folded into that GEMV: h = res_in +
// delta (delta may be NULL: h = res_in), written to res_out if that is not NULL
// (distinct from res_in and delta), and y = RMSNorm(h) . W.  Factored (exact ==
// false): computed as (W . (h * gamma)) / rms(h), so that no reduction precedes
// the staging; rounds differently from the unfolded step.  Exact: every workgroup
// forms sum(h^2) first and stages RMSNorm(h) as the RMSNorm kernel rounds it, so y
// is bitwise the RMSNorm kernel followed by the GEMV.  All fp16 vectors of K
// values, 16-byte aligned.
struct NormIn {
  const uint16_t* delta = nullptr;
  const uint16_t* res_in = nullptr;
  const uint16_t* gamma = nullptr;
  uint16_t* res_out = nullptr;
  float eps = 0.f;
  bool exact = false;
};

// y[i] for i < N of W [N][K] (glu: W has 2N rows and y[i] = silu_mul_h of rows i
// and N + i) with the input normalised as above; one K slice.  hipErrorInvalidValue
// when the staging does not fit a workgroup's LDS (K / 32 x 64 bytes, x 192 exact).
hipError_t launch_gemv_norm_in(const DeviceInfo& d, const uint32_t* words,
                               const uint16_t* scales, const NormIn& nin, uint16_t* y,
                               int64_t N, int64_t K, bool glu, hipStream_t s);

// h[i] = silu_mul_h(fp16(W[i] . x), fp16(W[F + i] . x)) for i < F, W having 2F
// rows; plan: the plan of the whole 2F-row GEMV, which needs splits == 1.
hipError_t launch_gemv_glu(const DeviceInfo& d, const uint32_t* words, const uint16_t* scales,
                           const uint16_t* x, uint16_t* h, int64_t F, int64_t K,
                           const GemvPlan& p, hipStream_t s);

}  // namespace q4
