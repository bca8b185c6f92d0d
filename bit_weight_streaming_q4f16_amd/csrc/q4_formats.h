// Format-variant GEMVs beside q4f16_1 that the entry point calls directly.
#pragma once

#include "q4_internal.h"

namespace q4 {

// y = W x at M = 1 in q3f16_1 (see include/q4f16.h); staged: 1 the words as
// 16-byte pieces through an LDS stage, 0 one 12-byte load per group, -1 chosen
// by size.  The results do not depend on it.
hipError_t launch_gemv_q3(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                          const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, int staged,
                          hipStream_t s);

// y = W x at M = 1 in the MLX affine 4-bit format, group 64 (q4_gemv.hip: the
// q4f16_1 GEMV with a scale and a bias per two of its groups); bf16 scales and
// biases (the pages' format) or fp16 ones.  K <= 32768.
hipError_t launch_gemv_affine(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                              const uint16_t* B, const uint16_t* X, uint16_t* Y, int64_t N,
                              int64_t K, bool bf16, hipStream_t s);

}  // namespace q4
