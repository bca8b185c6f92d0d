// GEMV for format variants beside q4f16_1 (everything-webgpu AI.md,
// quantization table), at M = 1, on the skeleton of the q4f16_1 kernels: a team
// of lanes per row, x staged once per workgroup in LDS, a DPP/lane-swap
// reduction.  Only the decode and the load pattern differ:
//   q3f16_1: a group is three words (12 bytes) holding 32 3-bit codes as one
//     96-bit value; weight = (q - 3) * s, s fp16 per 32 (k_gemv_q3).
//   q4f32_1: q4f16_1's words with fp32 scales; x and y fp32 (k_gemv_fmt): a lane
//     forms sum(q * x) per group in fp32 (codes converted exactly), and the zero
//     point enters through the group's sum of x, staged beside x:
//     (q - 7) * s summed = s * (sum q x - 7 sum x).
// The MLX affine format runs on the q4f16_1 GEMV itself (q4_gemv.hip).
#include "q4_formats.h"
#include "q4_device.h"

namespace q4 {
namespace {

enum : int { kQ3 = 1, kQ4F32 = 2 };

// Weights per group and words per group of a format.
template <int F> struct Fmt;
template <> struct Fmt<kQ4F32> { static constexpr int kGroup = 32, kWords = 4; };

// sum over group g of q * x; x from LDS planes xs4[j][g] = x[GS*g + 4j .. +3], so
// the lanes of a team (consecutive g) read consecutive 16-byte entries.  A
// word's even and odd nibbles are split into the bytes of two words, so that
// each code is converted by one byte-to-float instruction.
template <int F>
__device__ __forceinline__ float group_qx(const uint32_t (&w)[Fmt<F>::kWords],
                                          const float4* xs4, int G, int g) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int k = 0; k < Fmt<F>::kWords; ++k) {
    uint32_t ev = w[k] & 0x0F0F0F0Fu;          // codes 8k, 8k+2, 8k+4, 8k+6
    uint32_t od = (w[k] >> 4) & 0x0F0F0F0Fu;   // codes 8k+1, 8k+3, 8k+5, 8k+7
    // hide the known zero bits: with them the compiler turns a byte's shift and
    // mask into a 4-bit extract plus a conversion, not one v_cvt_f32_ubyteN
    asm volatile("" : "+v"(ev), "+v"(od));
    const float4 x0 = xs4[(2 * k) * G + g], x1 = xs4[(2 * k + 1) * G + g];
    a = __builtin_fmaf((float)(ev & 0xFFu), x0.x, a);
    b = __builtin_fmaf((float)(od & 0xFFu), x0.y, b);
    a = __builtin_fmaf((float)((ev >> 8) & 0xFFu), x0.z, a);
    b = __builtin_fmaf((float)((od >> 8) & 0xFFu), x0.w, b);
    a = __builtin_fmaf((float)((ev >> 16) & 0xFFu), x1.x, a);
    b = __builtin_fmaf((float)((od >> 16) & 0xFFu), x1.y, b);
    a = __builtin_fmaf((float)(ev >> 24), x1.z, a);
    b = __builtin_fmaf((float)(od >> 24), x1.w, b);
  }
  return a + b;
}

// Grid: workgroups striding over rows; a team of LPR lanes per row; lane i takes
// groups i, i + LPR, ...  LDS: x as fp32 planes of float4 [GS/4][G], then the sum
// of x per group [G].
template <int F, int LPR>
__global__ __launch_bounds__(kBlock) void k_gemv_fmt(const uint32_t* __restrict__ W,
                                                     const void* __restrict__ Sv,
                                                     const void* __restrict__ Xv,
                                                     void* __restrict__ Yv, int N, int K) {
  constexpr int GS = Fmt<F>::kGroup, NW = Fmt<F>::kWords;
  extern __shared__ float4 xs4[];
  const int G = K / GS;
  float* gsum = reinterpret_cast<float*>(xs4 + K / 4);
  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  auto chunk = [&](int c) {   // x[4c .. 4c + 3] as fp32
    if constexpr (F == kQ4F32) {
      return static_cast<const float4*>(Xv)[c];
    } else {
      const uint2 h = static_cast<const uint2*>(Xv)[c];
      return make_float4((float)bits<_Float16>((uint16_t)(h.x & 0xFFFFu)),
                         (float)bits<_Float16>((uint16_t)(h.x >> 16)),
                         (float)bits<_Float16>((uint16_t)(h.y & 0xFFFFu)),
                         (float)bits<_Float16>((uint16_t)(h.y >> 16)));
    }
  };
  // This thread's first PX chunks of x, then the first group of its team's first
  // row, are loaded before x is staged, without a branch (indices clamped; a
  // duplicate writes the same value, a group past the end is loaded and unused):
  // the compiler counts outstanding loads in order only through straight-line
  // code, so the staging then waits for x, not for the weights behind it.
  constexpr int PX = 4;
  float4 xp[PX];
#pragma unroll
  for (int j = 0; j < PX; ++j) {
    const int c = (int)threadIdx.x + j * kBlock;
    xp[j] = chunk(c < K / 4 ? c : K / 4 - 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int nf = team < N ? team : N - 1, gf = lane < G ? lane : G - 1;
  uint32_t wf[NW];
  {
    const uint32_t* wp = W + ((int64_t)nf * G + gf) * NW;
#pragma unroll
    for (int j = 0; j < NW; j += 4) {
      const uint4 v = load_nt(reinterpret_cast<const uint4*>(wp + j));
      wf[j] = v.x; wf[j + 1] = v.y; wf[j + 2] = v.z; wf[j + 3] = v.w;
    }
  }
  const float sf = static_cast<const float*>(Sv)[(int64_t)nf * G + gf];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < PX; ++j) {
    int c = (int)threadIdx.x + j * kBlock;
    c = c < K / 4 ? c : K / 4 - 1;
    xs4[(c % (GS / 4)) * G + c / (GS / 4)] = xp[j];
  }
  for (int c = threadIdx.x + PX * kBlock; c < K / 4; c += kBlock)   // 4 consecutive x per chunk
    xs4[(c % (GS / 4)) * G + c / (GS / 4)] = chunk(c);
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

  for (int n = team; n < N; n += nteams) {
    float acc = 0.f;
    int g1 = lane;
    if (n == team) {            // the group loaded before the staging
      if (lane < G) acc = __builtin_fmaf(sf, group_qx<F>(wf, xs4, G, lane) - 7.f * gsum[lane], acc);
      g1 = lane + LPR;
    }
    for (int g = g1; g < G; g += LPR) {
      uint32_t w[NW];
      const uint32_t* wp = W + ((int64_t)n * G + g) * NW;
#pragma unroll
      for (int j = 0; j < NW; j += 4) {
        const uint4 v = load_nt(reinterpret_cast<const uint4*>(wp + j));
        w[j] = v.x; w[j + 1] = v.y; w[j + 2] = v.z; w[j + 3] = v.w;
      }
      const float qx = group_qx<F>(w, xs4, G, g);
      const int64_t gi = (int64_t)n * G + g;
      const float s = static_cast<const float*>(Sv)[gi];
      acc = __builtin_fmaf(s, qx - 7.f * gsum[g], acc);
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

typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

// Grid: workgroups striding over rows, a team of LPR lanes per row.  A trip of a
// team covers 4 * LPR consecutive groups of its row (48 LPR bytes); lane i
// computes groups i, i + LPR, i + 2 LPR, i + 3 LPR of it.  Every load instruction
// reads one contiguous span per team (a lane taking four adjacent groups as
// three 16-byte loads made each instruction touch every cache line of the span,
// and streamed at two thirds of the rate).  Two ways to load:
//  * STAGED: three 16-byte loads per lane (lane i load j: bytes 16 (j LPR + i)),
//    the raw bytes through the wave's own LDS stage, from which lane i reads
//    its four groups (12-byte entries: consecutive lanes, consecutive banks).  A
//    wave's LDS operations complete in order, so the stage needs no barrier.
//  * otherwise: one 12-byte load per group.  Those stream a fifth slower than
//    16-byte ones, but the stage adds latency to every trip, which costs more
//    when a team has only a few trips.
// Loads go through a buffer resource based at the wave's first row (its teams
// hold consecutive rows), so offsets stay 32-bit and rows past the matrix read
// zero.  The next trip's loads are issued before a trip is computed, the first
// trip's before x is staged.  LDS: the pairs as uint4 at xq[c * G + g] (chunk c
// of group g; the lanes of a team read consecutive entries), the per-group
// correction [G] (rounded up to 16 bytes), then one 3 KB stage per wave.
template <int LPR, bool STAGED>
__global__ __launch_bounds__(kBlock) void k_gemv_q3(const uint32_t* __restrict__ W,
                                                    const uint16_t* __restrict__ S,
                                                    const uint4* __restrict__ X,
                                                    uint16_t* __restrict__ Y, int N, int K) {
  extern __shared__ uint4 xq[];
  const int G = K / 32;
  float* corr = reinterpret_cast<float*>(xq + 4 * G);
  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  const int T = (G + 4 * LPR - 1) / (4 * LPR);   // trips per row
  // this lane's places in its wave's stage: where it writes load j, where it
  // reads group t (in dwords)
  uint32_t* const stage = reinterpret_cast<uint32_t*>(xq + 4 * G + (G + 3) / 4) +
                          (threadIdx.x >> 6) * 768;
  uint32_t* const st_team = stage + ((threadIdx.x & 63) / LPR) * 12 * LPR;
  struct Trip {
    uint4 r[3];     // STAGED: the trip's bytes 16 (j LPR + lane) .. + 15
    u32x3_t w[4];   // otherwise: groups lane + t LPR of the trip
    uint32_t s[4];  // their scales
  };
  auto fetch = [&](Trip& f, int n, int tr) {
    const int n0 = __builtin_amdgcn_readfirstlane(n);   // the wave's first row
    const int64_t left = N > n0 ? (int64_t)(N - n0) * G : 0;
    const uint32_t nw = left * 12 < 0xFFFFFFF0ll ? (uint32_t)(left * 12) : 0xFFFFFFF0u;
    const uint32_t ns = left * 2 < 0xFFFFFFF0ll ? (uint32_t)(left * 2) : 0xFFFFFFF0u;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(W + (int64_t)n0 * G * 3), 0, (int)nw, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(S + (int64_t)n0 * G), 0, (int)ns, kRsrcFlags);
    const int gt = (n - n0) * G + tr * 4 * LPR;   // the trip's first group
    if constexpr (STAGED) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(
            rw, gt * 12 + (j * LPR + lane) * 16, 0, kNonTemporal);
        f.r[j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        f.w[t] = __builtin_amdgcn_raw_buffer_load_b96(rw, (gt + t * LPR + lane) * 12, 0,
                                                      kNonTemporal);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      f.s[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, (gt + t * LPR + lane) * 2, 0, 0);
  };
  // x is loaded before the first trip's weights, and without a branch (indices
  // clamped, a duplicate writes the same value): the compiler counts outstanding
  // loads in order only through straight-line code, so the staging then waits for
  // x, not for the weights behind it.  Thread t stages blocks t and t + 256 of x
  // and forms the correction of group t from its four blocks.
  auto pair = [](uint4 v) {
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.z << 16);
    o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o.z = (v.y & 0xFFFFu) | (v.w << 16);
    o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return o;
  };
  // 2^E + 3 for the codes 8c .. 8c+7 of a chunk
  constexpr float kOff[8] = {67.f, 11.f, 67.f, 11.f, 1027.f, 131.f, 1027.f, 131.f};
  auto correction = [&](const uint4 (&v4)[4]) {
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t hw[4] = {v4[c].x, v4[c].y, v4[c].z, v4[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        t = __builtin_fmaf(kOff[i], (float)bits<_Float16>((uint16_t)(hw[i / 2] >> (16 * (i & 1)))),
                           t);
    }
    return t;
  };
  const int e0 = (int)threadIdx.x < 4 * G ? (int)threadIdx.x : 4 * G - 1;
  const int e1 = (int)threadIdx.x + kBlock < 4 * G ? (int)threadIdx.x + kBlock : 4 * G - 1;
  const int gx = (int)threadIdx.x < G ? (int)threadIdx.x : G - 1;
  const uint4 x0 = X[e0], x1 = X[e1];
  uint4 xg[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) xg[c] = X[4 * gx + c];
  __builtin_amdgcn_sched_barrier(0);
  Trip cur;
  int n = team, tr = 0;
  fetch(cur, n, 0);
  __builtin_amdgcn_sched_barrier(0);
  xq[(e0 & 3) * G + (e0 >> 2)] = pair(x0);
  xq[(e1 & 3) * G + (e1 >> 2)] = pair(x1);
  for (int e = threadIdx.x + 2 * kBlock; e < 4 * G; e += kBlock)   // e: x[8e .. 8e+7]
    xq[(e & 3) * G + (e >> 2)] = pair(X[e]);
  corr[gx] = correction(xg);
  for (int g = threadIdx.x + kBlock; g < G; g += kBlock) {
    uint4 v4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v4[c] = X[4 * g + c];
    corr[g] = correction(v4);
  }
  __syncthreads();

  uint32_t ma = kQ3MaskA, mb = kQ3MaskB;
  asm volatile("" : "+v"(ma), "+v"(mb));
  float acc = 0.f;
  // Compute the trip held in `use` after issuing the next one into `fill`; two
  // buffers taken in turn, so no register copy waits for the loads in flight.
  auto step = [&](Trip& use, Trip& fill) {
    int n2 = n, tr2 = tr + 1;
    if (tr2 == T) {
      tr2 = 0;
      n2 += nteams;
    }
    uint32_t w[4][3];
    if constexpr (STAGED) {
      // the stage is read by other lanes: keep its writes and reads in program order
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < 3; ++j)
        *reinterpret_cast<uint4*>(st_team + 4 * (j * LPR + lane)) = use.r[j];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int k = 0; k < 3; ++k) w[t][k] = st_team[3 * (t * LPR + lane) + k];
      asm volatile("" ::: "memory");
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int k = 0; k < 3; ++k) w[t][k] = use.w[t][k];
    }
    fetch(fill, n2, tr2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int g = tr * 4 * LPR + t * LPR + lane;
      if (g < G) {
        const float d = q3_group_dot(w[t][0], w[t][1], w[t][2], xq + g, G, ma, mb);
        const float sc = (float)bits<_Float16>((uint16_t)use.s[t]);
        acc = __builtin_fmaf(sc, d - corr[g], acc);
      }
    }
    if (tr == T - 1) {
      acc = team_sum<LPR>(acc);
      if (lane == 0) Y[n] = bits<uint16_t>((_Float16)acc);
      acc = 0.f;
    }
    n = n2;
    tr = tr2;
  };
  Trip other;
  while (n < N) {
    step(cur, other);
    if (n >= N) break;
    step(other, cur);
  }
}

template <int LPR, bool STAGED>
hipError_t launch_q3_kern(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                          const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, int64_t blocks,
                          hipStream_t s) {
  const int64_t G = K / 32;
  const size_t lds =
      (size_t)G * 64 + (size_t)(G + 3) / 4 * 16 + (STAGED ? (kBlock / 64) * 3072 : 0);
  auto kern = k_gemv_q3<LPR, STAGED>;
  if (lds > 65536)
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
      return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s, W, S,
                     reinterpret_cast<const uint4*>(X), Y, (int)N, (int)K);
  return hipGetLastError();
}

// staged < 0: the staged loads once a team has at least eight trips (A/B on one
// GPU: a 262144 x 3072 GEMV 64.8 -> 59.5 us staged; qkv- and LM-head-sized ones,
// one or two rows per team, 7.6 -> 8.5 us).
template <int LPR>
hipError_t launch_q3_lpr(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                         const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, int staged,
                         hipStream_t s) {
  const int64_t G = K / 32;
  const int64_t rows_per_block = kBlock / LPR;
  int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
  if (blocks > (int64_t)d.cus * 8) blocks = (int64_t)d.cus * 8;
  const int64_t teams = blocks * rows_per_block;
  const int64_t trips = (N + teams - 1) / teams * ((G + 4 * LPR - 1) / (4 * LPR));
  if (staged > 0 || (staged < 0 && trips >= 8))
    return launch_q3_kern<LPR, true>(d, W, S, X, Y, N, K, blocks, s);
  return launch_q3_kern<LPR, false>(d, W, S, X, Y, N, K, blocks, s);
}

// Lanes per row: a power of two with at most four trips per row.
hipError_t launch_q3(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                     const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, int staged,
                     hipStream_t s) {
  const int64_t G = K / 32;
  if (G <= 64) return launch_q3_lpr<4>(d, W, S, X, Y, N, K, staged, s);
  if (G <= 128) return launch_q3_lpr<8>(d, W, S, X, Y, N, K, staged, s);
  if (G <= 256) return launch_q3_lpr<16>(d, W, S, X, Y, N, K, staged, s);
  if (G <= 512) return launch_q3_lpr<32>(d, W, S, X, Y, N, K, staged, s);
  return launch_q3_lpr<64>(d, W, S, X, Y, N, K, staged, s);
}

template <int F, int LPR>
hipError_t launch_fmt_lpr(const DeviceInfo& d, const uint32_t* W, const void* S, const void* X,
                          void* Y, int64_t N, int64_t K, hipStream_t s) {
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
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kBlock), lds, s, W, S, X, Y, (int)N,
                     (int)K);
  return hipGetLastError();
}

template <int F>
hipError_t launch_fmt(const DeviceInfo& d, const uint32_t* W, const void* S, const void* X,
                      void* Y, int64_t N, int64_t K, hipStream_t s) {
  // lanes per row: a power of two with at most four groups per lane
  const int64_t G = K / Fmt<F>::kGroup;
  if (G <= 16) return launch_fmt_lpr<F, 4>(d, W, S, X, Y, N, K, s);
  if (G <= 32) return launch_fmt_lpr<F, 8>(d, W, S, X, Y, N, K, s);
  if (G <= 64) return launch_fmt_lpr<F, 16>(d, W, S, X, Y, N, K, s);
  if (G <= 128) return launch_fmt_lpr<F, 32>(d, W, S, X, Y, N, K, s);
  return launch_fmt_lpr<F, 64>(d, W, S, X, Y, N, K, s);
}

}  // namespace

hipError_t launch_gemv_q3(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                          const uint16_t* X, uint16_t* Y, int64_t N, int64_t K, int staged,
                          hipStream_t s) {
  return launch_q3(d, W, S, X, Y, N, K, staged, s);
}

hipError_t launch_gemv_format(const DeviceInfo& d, int format, const uint32_t* W, const void* S,
                              const uint16_t* B, const void* X, void* Y, int64_t N, int64_t K,
                              hipStream_t s) {
  switch (format) {
    case kQ3:
      return launch_q3(d, W, static_cast<const uint16_t*>(S), static_cast<const uint16_t*>(X),
                       static_cast<uint16_t*>(Y), N, K, -1, s);
    case kQ4F32: return launch_fmt<kQ4F32>(d, W, S, X, Y, N, K, s);
    default:
      return launch_gemv_affine(d, W, static_cast<const uint16_t*>(S), B,
                                static_cast<const uint16_t*>(X), static_cast<uint16_t*>(Y), N, K,
                                format == 3, s);
  }
}

}  // namespace q4
