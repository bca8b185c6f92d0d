// GEMV for the format variants beside q4f16_1 (everything-webgpu AI.md,
// quantization table; Zero TVM documentation, the MLX affine checkpoints), at
// M = 1, on the skeleton of the q4f16_1 kernels: a team of lanes per row, x
// staged once per workgroup in LDS, each lane taking every LPR-th group of its
// row, a DPP/lane-swap reduction.  Only the decode differs:
//   q3f16_1: a group is three words (12 bytes) holding 32 3-bit codes as one
//     96-bit value; weight = (q - 3) * s, s fp16 per 32.
//   q4f32_1: q4f16_1's words with fp32 scales; x and y fp32.
//   af4g64 (MLX affine): q4f16_1's nibble order, fp16 scale s and bias b per 64
//     weights; weight = s * q + b.
// Per group a lane forms sum(q * x) in fp32 (codes converted exactly), and the
// zero point or bias enters through the group's sum of x, staged beside x:
// (q - z) * s summed = s * (sum q x - z * sum x); s * q + b summed = s * sum q x
// + b * sum x.
#include "q4_internal.h"

namespace q4 {
namespace {

template <typename T, typename F>
__device__ __forceinline__ T bits(F v) {
  return __builtin_bit_cast(T, v);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return bits<float>(__builtin_amdgcn_update_dpp(0, bits<int>(v), CTRL, 0xF, 0xF, true));
}

template <int LPR>
__device__ __forceinline__ float team_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  if constexpr (LPR >= 8) v += dpp<0x141>(v);
  if constexpr (LPR >= 16) v += dpp<0x140>(v);
  if constexpr (LPR >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  if constexpr (LPR >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  return v;
}

enum : int { kQ3 = 1, kQ4F32 = 2, kAF4 = 3 };

// Weights per group and words per group of a format.
template <int F> struct Fmt;
template <> struct Fmt<kQ3> { static constexpr int kGroup = 32, kWords = 3; };
template <> struct Fmt<kQ4F32> { static constexpr int kGroup = 32, kWords = 4; };
template <> struct Fmt<kAF4> { static constexpr int kGroup = 64, kWords = 8; };

// code i (0 .. kGroup-1) of a group's words
template <int F>
__device__ __forceinline__ float code_at(const uint32_t (&w)[Fmt<F>::kWords], int i) {
  if constexpr (F == kQ3) {
    // codes 0..20 lie in bits 0..62 of w0 | w1 << 32, codes 21..31 in bits 31..63
    // of w1 | w2 << 32
    const uint64_t v = i <= 20 ? ((uint64_t)w[0] | ((uint64_t)w[1] << 32))
                               : ((uint64_t)w[1] | ((uint64_t)w[2] << 32));
    return (float)((uint32_t)(v >> (i <= 20 ? 3 * i : 3 * i - 32)) & 7u);
  } else {
    return (float)((w[i / 8] >> (4 * (i % 8))) & 0xFu);
  }
}

// sum over group g of q * x; x from LDS planes xs4[j][g] = x[GS*g + 4j .. +3], so
// the lanes of a team (consecutive g) read consecutive 16-byte entries
template <int F>
__device__ __forceinline__ float group_qx(const uint32_t (&w)[Fmt<F>::kWords],
                                          const float4* xs4, int G, int g) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int j = 0; j < Fmt<F>::kGroup / 4; ++j) {
    const float4 xv = xs4[j * G + g];
    a = __builtin_fmaf(code_at<F>(w, 4 * j), xv.x, a);
    b = __builtin_fmaf(code_at<F>(w, 4 * j + 1), xv.y, b);
    a = __builtin_fmaf(code_at<F>(w, 4 * j + 2), xv.z, a);
    b = __builtin_fmaf(code_at<F>(w, 4 * j + 3), xv.w, b);
  }
  return a + b;
}

// Grid: workgroups striding over rows; a team of LPR lanes per row; lane i takes
// groups i, i + LPR, ...  LDS: x as fp32 planes of float4 [GS/4][G], then the sum
// of x per group [G].
template <int F, int LPR>
__global__ __launch_bounds__(kBlock) void k_gemv_fmt(const uint32_t* __restrict__ W,
                                                     const void* __restrict__ Sv,
                                                     const uint16_t* __restrict__ Bv,
                                                     const void* __restrict__ Xv,
                                                     void* __restrict__ Yv, int N, int K) {
  constexpr int GS = Fmt<F>::kGroup, NW = Fmt<F>::kWords;
  extern __shared__ float4 xs4[];
  const int G = K / GS;
  float* gsum = reinterpret_cast<float*>(xs4 + K / 4);
  for (int c = threadIdx.x; c < K / 4; c += kBlock) {   // 4 consecutive x per chunk
    float4 v;
    if constexpr (F == kQ4F32) {
      v = static_cast<const float4*>(Xv)[c];
    } else {
      const uint2 h = static_cast<const uint2*>(Xv)[c];
      v = make_float4((float)bits<_Float16>((uint16_t)(h.x & 0xFFFFu)),
                      (float)bits<_Float16>((uint16_t)(h.x >> 16)),
                      (float)bits<_Float16>((uint16_t)(h.y & 0xFFFFu)),
                      (float)bits<_Float16>((uint16_t)(h.y >> 16)));
    }
    xs4[(c % (GS / 4)) * G + c / (GS / 4)] = v;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += kBlock) {
    float t = 0.f;
    for (int j = 0; j < GS / 4; ++j) {
      const float4 v = xs4[j * G + g];
      t += (v.x + v.y) + (v.z + v.w);
    }
    gsum[g] = t;
  }
  __syncthreads();

  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  for (int n = team; n < N; n += nteams) {
    float acc = 0.f;
    for (int g = lane; g < G; g += LPR) {
      uint32_t w[NW];
      const uint32_t* wp = W + ((int64_t)n * G + g) * NW;
      if constexpr (NW == 3) {
#pragma unroll
        for (int j = 0; j < 3; ++j) w[j] = __builtin_nontemporal_load(wp + j);
      } else {
#pragma unroll
        for (int j = 0; j < NW; j += 4) {
          const uint4 v = load_nt(reinterpret_cast<const uint4*>(wp + j));
          w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
        }
      }
      const float qx = group_qx<F>(w, xs4, G, g);
      const int64_t gi = (int64_t)n * G + g;
      if constexpr (F == kQ3) {
        const float s = (float)bits<_Float16>(static_cast<const uint16_t*>(Sv)[gi]);
        acc = __builtin_fmaf(s, qx - 3.f * gsum[g], acc);
      } else if constexpr (F == kQ4F32) {
        const float s = static_cast<const float*>(Sv)[gi];
        acc = __builtin_fmaf(s, qx - 7.f * gsum[g], acc);
      } else {
        const float s = (float)bits<_Float16>(static_cast<const uint16_t*>(Sv)[gi]);
        const float b = (float)bits<_Float16>(Bv[gi]);
        acc = __builtin_fmaf(s, qx, __builtin_fmaf(b, gsum[g], acc));
      }
    }
    acc = team_sum<LPR>(acc);
    if (lane == 0) {
      if (F == kQ4F32)
        static_cast<float*>(Yv)[n] = acc;
      else
        static_cast<uint16_t*>(Yv)[n] = bits<uint16_t>((_Float16)acc);
    }
  }
}

template <int F, int LPR>
hipError_t launch_fmt_lpr(const DeviceInfo& d, const uint32_t* W, const void* S,
                          const uint16_t* B, const void* X, void* Y, int64_t N, int64_t K,
                          hipStream_t s) {
  const int G = (int)(K / Fmt<F>::kGroup);
  const size_t lds = (size_t)(K + G) * sizeof(float);
  auto kern = k_gemv_fmt<F, LPR>;
  if (lds > 65536)
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
      return e;
  const int64_t rows_per_block = kBlock / LPR;
  int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
  if (blocks > (int64_t)d.cus * 8) blocks = (int64_t)d.cus * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s, W, S, B, X, Y, (int)N,
                     (int)K);
  return hipGetLastError();
}

template <int F>
hipError_t launch_fmt(const DeviceInfo& d, const uint32_t* W, const void* S, const uint16_t* B,
                      const void* X, void* Y, int64_t N, int64_t K, hipStream_t s) {
  // lanes per row: a power of two with at most four groups per lane
  const int64_t G = K / Fmt<F>::kGroup;
  if (G <= 16) return launch_fmt_lpr<F, 4>(d, W, S, B, X, Y, N, K, s);
  if (G <= 32) return launch_fmt_lpr<F, 8>(d, W, S, B, X, Y, N, K, s);
  if (G <= 64) return launch_fmt_lpr<F, 16>(d, W, S, B, X, Y, N, K, s);
  if (G <= 128) return launch_fmt_lpr<F, 32>(d, W, S, B, X, Y, N, K, s);
  return launch_fmt_lpr<F, 64>(d, W, S, B, X, Y, N, K, s);
}

}  // namespace

hipError_t launch_gemv_format(const DeviceInfo& d, int format, const uint32_t* W, const void* S,
                              const uint16_t* B, const void* X, void* Y, int64_t N, int64_t K,
                              hipStream_t s) {
  switch (format) {
    case kQ3: return launch_fmt<kQ3>(d, W, S, B, X, Y, N, K, s);
    case kQ4F32: return launch_fmt<kQ4F32>(d, W, S, B, X, Y, N, K, s);
    default: return launch_fmt<kAF4>(d, W, S, B, X, Y, N, K, s);
  }
}

}  // namespace q4
