// The feed-forward glue of the decode loop (Zero TVM documentation, "Decode
// loop") folded into the gate/up GEMV, so that a decode step launches one kernel
// fewer per block: on this GPU every kernel boundary costs a few microseconds
// whatever the kernel does.  One team computes row i of gate and row i of up
// (rows i and F + i of the gate_up matrix) and writes silu_mul_h(fp16(gate),
// fp16(up)) -- bitwise what the GEMV followed by the glue kernel writes.
#pragma once

#include "q4_internal.h"

namespace q4 {

// h[i] = silu_mul_h(fp16(W[i] . x), fp16(W[F + i] . x)) for i < F, W having 2F
// rows; plan: the plan of the whole 2F-row GEMV, which needs splits == 1.
hipError_t launch_gemv_glu(const DeviceInfo& d, const uint32_t* words, const uint16_t* scales,
                           const uint16_t* x, uint16_t* h, int64_t F, int64_t K,
                           const GemvPlan& p, hipStream_t s);

}  // namespace q4
