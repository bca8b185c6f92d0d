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

// q3f16_1 when K % 128 == 0 and the words are 16-byte aligned: a lane takes
// four consecutive groups (48 bytes, three 128-bit loads) per trip, and the
// codes become fp16 pairs without extracting them one by one.  A 32-bit window
// of the group's 96-bit value, taken at bit 3i - 4 (one shift or funnel shift),
// holds code i at bits 4-6, code i+1 at 7-9, code i+4 at 16-18 and code i+5 at
// 19-21.  Masking two of those fields and OR-ing in an exponent chosen per
// field so that the field's lowest bit has place value 1 gives fp16 values
// 2^E + q exactly (E = 6, 3, 10, 7 for the four fields), one AND-OR per pair;
// v_dot2_f32_f16 multiplies a pair by the matching x pair.  Per group the sum
// of (2^E + 3) * x over its codes is staged beside x and subtracted once, which
// leaves sum (q - 3) * x.  Windows at i = 0, 2, 8, 10, 16, 18, 24, 26 cover the
// 32 codes as the pairs (i, i+4), (i+1, i+5).
constexpr uint32_t kQ3MaskA = 0x00070070u, kQ3MaskB = 0x00380380u;
constexpr uint32_t kQ3ExpA = 0x64005400u, kQ3ExpB = 0x58004800u;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Sum over one group of (2^E + q) * x.  xq: x of the group as four chunks of
// four pairs, chunk c at xq[c * cstride] holding the pairs (x[8c+p], x[8c+p+4]).
// ma, mb: kQ3MaskA and kQ3MaskB held in registers (an instruction with three
// operands takes no literal constant, and two literals would split each AND-OR
// into two instructions).
__device__ __forceinline__ float q3_group_dot(uint32_t w0, uint32_t w1, uint32_t w2,
                                              const uint4* xq, int cstride, uint32_t ma,
                                              uint32_t mb) {
  const uint32_t v[8] = {w0 << 4,
                         __builtin_amdgcn_alignbit(w1, w0, 2),
                         __builtin_amdgcn_alignbit(w1, w0, 20),
                         __builtin_amdgcn_alignbit(w1, w0, 26),
                         __builtin_amdgcn_alignbit(w2, w1, 12),
                         __builtin_amdgcn_alignbit(w2, w1, 18),
                         w2 >> 4,
                         w2 >> 10};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 xv = xq[c * cstride];
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & ma) | kQ3ExpA), bits<h2_t>(xv.x), a,
                               false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c] & mb) | kQ3ExpB), bits<h2_t>(xv.y), b,
                               false);
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & ma) | kQ3ExpA),
                               bits<h2_t>(xv.z), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v[2 * c + 1] & mb) | kQ3ExpB),
                               bits<h2_t>(xv.w), b, false);
  }
  return a + b;
}

// LDS: the pairs as uint4 at xq[(c * 4 + t) * Q + u] for group g = 4u + t, chunk
// c (so the lanes of a team, consecutive u, read consecutive 16-byte entries),
// then the per-group correction [G].
template <int LPR>
__global__ __launch_bounds__(kBlock) void k_gemv_q3(const uint4* __restrict__ W,
                                                    const uint16_t* __restrict__ S,
                                                    const uint4* __restrict__ X,
                                                    uint16_t* __restrict__ Y, int N, int K) {
  extern __shared__ uint4 xq[];
  const int G = K / 32, Q = G / 4;
  float* corr = reinterpret_cast<float*>(xq + 4 * G);
  for (int e = threadIdx.x; e < 4 * G; e += kBlock) {   // e: x[8e .. 8e+7]
    const uint4 v = X[e];
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    const int g = e >> 2, c = e & 3;
    xq[(c * 4 + (g & 3)) * Q + (g >> 2)] = o;
  }
  // 2^E + 3 for the codes 8c .. 8c+7 of a chunk
  constexpr float kOff[8] = {67.f, 11.f, 67.f, 11.f, 1027.f, 131.f, 1027.f, 131.f};
  for (int g = threadIdx.x; g < G; g += kBlock) {
    float t = 0.f;
    for (int c = 0; c < 4; ++c) {
      const uint4 v = X[4 * g + c];
      const uint32_t hw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        t = __builtin_fmaf(kOff[i], (float)bits<_Float16>((uint16_t)(hw[i / 2] >> (16 * (i & 1)))),
                           t);
    }
    corr[g] = t;
  }
  __syncthreads();

  uint32_t ma = kQ3MaskA, mb = kQ3MaskB;
  asm volatile("" : "+v"(ma), "+v"(mb));
  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  for (int n = team; n < N; n += nteams) {
    float acc = 0.f;
    for (int u = lane; u < Q; u += LPR) {
      const uint4* wp = W + ((int64_t)n * Q + u) * 3;   // groups 4u .. 4u+3: 12 words
      const uint4 a = load_nt(wp), b = load_nt(wp + 1), c = load_nt(wp + 2);
      const uint2 sv = *reinterpret_cast<const uint2*>(S + (int64_t)n * G + 4 * u);
      const uint32_t w[12] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w};
      const uint32_t sw[2] = {sv.x, sv.y};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float d =
            q3_group_dot(w[3 * t], w[3 * t + 1], w[3 * t + 2], xq + t * Q + u, 4 * Q, ma, mb);
        const float sc = (float)bits<_Float16>((uint16_t)(sw[t / 2] >> (16 * (t & 1))));
        acc = __builtin_fmaf(sc, d - corr[4 * u + t], acc);
      }
    }
    acc = team_sum<LPR>(acc);
    if (lane == 0) Y[n] = bits<uint16_t>((_Float16)acc);
  }
}

template <int LPR>
hipError_t launch_q3_lpr(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                         const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, hipStream_t s) {
  const int64_t G = K / 32;
  const size_t lds = (size_t)G * 64 + (size_t)G * sizeof(float);
  auto kern = k_gemv_q3<LPR>;
  if (lds > 65536)
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
      return e;
  const int64_t rows_per_block = kBlock / LPR;
  int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
  if (blocks > (int64_t)d.cus * 8) blocks = (int64_t)d.cus * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s,
                     reinterpret_cast<const uint4*>(W), S, reinterpret_cast<const uint4*>(X), Y,
                     (int)N, (int)K);
  return hipGetLastError();
}

// K % 128 == 0, W 16-byte and S 8-byte aligned.  Lanes per row: a power of two
// with at most four trips of four groups per lane.
hipError_t launch_q3(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                     const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, hipStream_t s) {
  const int64_t Q = K / 128;
  if (Q <= 16) return launch_q3_lpr<4>(d, W, S, X, Y, N, K, s);
  if (Q <= 32) return launch_q3_lpr<8>(d, W, S, X, Y, N, K, s);
  if (Q <= 64) return launch_q3_lpr<16>(d, W, S, X, Y, N, K, s);
  if (Q <= 128) return launch_q3_lpr<32>(d, W, S, X, Y, N, K, s);
  return launch_q3_lpr<64>(d, W, S, X, Y, N, K, s);
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
    case kQ3:
      if (K % 128 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
          reinterpret_cast<uintptr_t>(S) % 8 == 0)
        return launch_q3(d, W, static_cast<const uint16_t*>(S), static_cast<const uint16_t*>(X),
                         static_cast<uint16_t*>(Y), N, K, s);
      return launch_fmt<kQ3>(d, W, S, B, X, Y, N, K, s);
    case kQ4F32: return launch_fmt<kQ4F32>(d, W, S, B, X, Y, N, K, s);
    default: return launch_fmt<kAF4>(d, W, S, B, X, Y, N, K, s);
  }
}

}  // namespace q4
