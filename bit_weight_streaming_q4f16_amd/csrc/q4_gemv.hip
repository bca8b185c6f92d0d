// q4f16_1 GEMV kernels for gfx950 (CDNA4, wave64).
//
// y[n] = sum_k (q[n][k] - 7) * s[n][k/32] * x[k]   (Zero TVM documentation,
// "Q4F16 quantization format"; fp32 accumulation as its correctness fixes ask).
//
// Decode is bandwidth-bound (everything-webgpu AI.md: time per token scales with
// weight bytes; the generated GEMV lost most of its speed to a barrier-heavy
// reduction over too little work per thread).  The design here follows that:
//  * weights stream with 128-bit non-temporal loads; one dwordx4 is four words,
//    i.e. exactly one 32-weight group, and its scale is one fp16;
//  * x is staged once per workgroup in LDS, already permuted to the order in
//    which the dequantised nibble pairs come out, in four planes so that lanes
//    reading consecutive groups hit consecutive LDS banks;
//  * dequantisation is exact and cheap: OR-ing a nibble pair into the mantissa
//    of two fp16 values with exponent 2^10 (nibbles at bits 0-3 and 16-19) or
//    2^6 (bits 4-7 and 20-23, whose place value 16 matches that exponent's ulp
//    of 1/16) gives 1024 + q or 64 + q exactly; one packed fp16 subtraction
//    gives q - 7 exactly; v_dot2_f32_f16 multiplies a pair by the matching x
//    pair and accumulates in fp32; the scale is applied once per group;
//  * each row's lanes reduce with DPP and lane-swap instructions, no LDS and no
//    barrier (the page's fix: reduce across lanes without workgroup barriers);
//  * a split-K variant writes fp32 partials per K slice; a second pass adds
//    them in ascending slice order, so results are deterministic;
//  * small M (2..8) uses MFMA: v_mfma_f32_16x16x32_f16 covers 16 rows by one
//    32-weight group, so the per-group scale is applied exactly to its result.
#include "q4_formats.h"
#include "q4_fused.h"
#include "q4_device.h"

namespace q4 {
namespace {

// One word -> four fp16 pairs (q0-7, q4-7) (q1-7, q5-7) (q2-7, q6-7) (q3-7, q7-7),
// all exact.
__device__ __forceinline__ void dequant_word(uint32_t w, h2_t (&q)[4]) {
  const uint32_t w8 = w >> 8;
  const h2_t c1031 = {(_Float16)-1031.0f, (_Float16)-1031.0f};
  const h2_t c71 = {(_Float16)-71.0f, (_Float16)-71.0f};
  q[0] = bits<h2_t>((w & 0x000F000Fu) | 0x64006400u) + c1031;
  q[1] = bits<h2_t>((w & 0x00F000F0u) | 0x54005400u) + c71;
  q[2] = bits<h2_t>((w8 & 0x000F000Fu) | 0x64006400u) + c1031;
  q[3] = bits<h2_t>((w8 & 0x00F000F0u) | 0x54005400u) + c71;
}

// sum over one 32-weight group of (q - 7) * x, fp32.  xs holds four planes of
// gc pair-ordered blocks: plane j, entry g = x of word j of group g.
__device__ __forceinline__ float group_dot(uint4 w, const uint4* xs, int gc, int g) {
  const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 xv = xs[j * gc + g];
    h2_t q[4];
    dequant_word(wj[j], q);
    a = __builtin_amdgcn_fdot2(q[0], bits<h2_t>(xv.x), a, false);
    b = __builtin_amdgcn_fdot2(q[1], bits<h2_t>(xv.y), b, false);
    a = __builtin_amdgcn_fdot2(q[2], bits<h2_t>(xv.z), a, false);
    b = __builtin_amdgcn_fdot2(q[3], bits<h2_t>(xv.w), b, false);
  }
  return a + b;
}

// K slice s of G groups split `splits` ways: [G*s/splits, G*(s+1)/splits).
__host__ __device__ __forceinline__ int slice_begin(int G, int splits, int s) {
  return (int)((int64_t)G * s / splits);
}

// ---------------------------------------------------------------- M == 1 ---
// Grid: x = workgroups striding over rows, y = K slice.  A team of LPR lanes owns
// a row at a time; lane i of the team takes groups i, i + LPR, ... of the slice,
// UNR of them per trip (loads first, then arithmetic; the launch picks UNR so that
// a slice is one trip).  Out-of-range groups load the slice's last group again and
// are discarded by a select.  A team's first loads are issued before x is staged
// (weights do not depend on x), so the two round trips overlap.  The next row's
// loads go out as soon as a row's arithmetic is done.
//
// Modes: kPlain writes y (or split-K partials); kGlu (q4_fused.h) computes rows
// i and F + i (F = N, the matrix has 2N rows) and writes silu_mul_h of the two
// rounded results; kAffineB (q4_formats.h; the MLX affine 4-bit format of the
// Splash models page, "MLX targets": the same nibble layout, one bf16 scale s
// and bf16 bias b per 64 weights, i.e. per two 16-byte groups) adds
// s * sum((q - 7) x) + (b + 7 s) * sum(x) per 32 weights, the sums of x staged
// beside x; kAffine is the same with fp16 scales and biases.  Both need one
// slice.  kPlainNorm and kGluNorm (q4_fused.h) are kPlain and kGlu
// with the residual add and RMSNorm of their input folded in, factored so that no
// reduction precedes the staging: x = h * gamma is staged (h = res_in + delta,
// rounded to fp16 as the RMSNorm kernel rounds it, and written to res_out by
// workgroup 0), sum(h^2) is formed alongside, and every output is scaled by
// 1 / sqrt(sum(h^2) / K + eps) before its rounding; with nin.exact they stage
// RMSNorm(h) itself instead, formed as the RMSNorm kernel forms it (h and gamma
// parked in LDS beside x while the workgroup sums h^2), and scale nothing, so the
// outputs are bitwise those of the RMSNorm kernel followed by kPlain or kGlu.
// They need one slice.
enum : int { kPlain = 0, kGlu = 1, kAffine = 2, kPlainNorm = 3, kGluNorm = 4, kAffineB = 5 };

// A bf16 bit pattern is the upper half of the fp32 with the same value.
__device__ __forceinline__ float bf16_to_float(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

template <int LPR, int UNR, int MODE>
__global__ __launch_bounds__(kBlock) void k_gemv_m1(const uint4* __restrict__ W,
                                                    const uint16_t* __restrict__ S,
                                                    const uint16_t* __restrict__ Bq,
                                                    const uint4* __restrict__ X,
                                                    uint16_t* __restrict__ Y,
                                                    float* __restrict__ P, int N, int G,
                                                    int splits, NormIn nin) {
  extern __shared__ uint4 xs[];
  __shared__ float ssw[kBlock / 64];
  constexpr bool kAff = MODE == kAffine || MODE == kAffineB;
  // scale (and bias) of a group as fp32
  auto sval = [](uint16_t h) { return MODE == kAffineB ? bf16_to_float(h) : half_to_float(h); };
  constexpr bool kNin = MODE == kPlainNorm || MODE == kGluNorm;
  const int split = blockIdx.y;
  const int g0 = slice_begin(G, splits, split);
  const int gc = slice_begin(G, splits, split + 1) - g0;
  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  constexpr int R = MODE == kGlu || MODE == kGluNorm ? 2 : 1;   // rows per team and output
  uint4 wv[R][UNR];
  uint16_t sv[R][UNR], bv[R][UNR];
  auto issue = [&](int n, int t0) {          // trip t0 of output n
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int64_t row = n + (int64_t)q * N;
      const uint4* wr = W + row * G + g0;
      const uint16_t* sr = kAff ? S + row * (G / 2) : S + row * G + g0;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        int g = t0 + u * LPR + lane;
        g = g < gc ? g : gc - 1;
        wv[q][u] = load_nt(wr + g);
        sv[q][u] = sr[kAff ? g >> 1 : g];
        if constexpr (kAff) bv[q][u] = Bq[row * (G / 2) + (g >> 1)];
      }
    }
  };
  int n = team;
  // Thread t stages blocks of 8 values t, t + 256, ... (kNin: the RMSNorm kernel's
  // order; one slice, g0 == 0 and gc == G).  Its first PRE blocks (kNin: residual,
  // delta and gamma) are loaded before the weights, and both without a branch
  // (indices clamped, surplus values unused): the compiler counts outstanding loads
  // in order only through straight-line code, so the staging then waits for its
  // own loads, not for the weights behind them.
  constexpr int PRE = kNin ? 2 : 4;
  const uint4* const nres = reinterpret_cast<const uint4*>(nin.res_in);
  const uint4* const ndel = reinterpret_cast<const uint4*>(nin.delta);
  const uint4* const ngam = reinterpret_cast<const uint4*>(nin.gamma);
  uint4 pr[PRE], pd[PRE], pg[PRE];
  // kAff: the four blocks of this thread's group (clamped) for the sums of x
  uint4 px[kAff ? 4 : 1];
  if constexpr (kAff) {
    const int g = (int)threadIdx.x < gc ? (int)threadIdx.x : gc - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) px[j] = X[(int64_t)(g0 + g) * 4 + j];
  }
#pragma unroll
  for (int j = 0; j < PRE; ++j) {
    int e = threadIdx.x + j * kBlock;
    e = e < 4 * gc ? e : 4 * gc - 1;
    if constexpr (kNin) {
      pr[j] = nres[e];
      pd[j] = (ndel ? ndel : nres)[e];
      pg[j] = ngam[e];
    } else {
      pr[j] = X[(int64_t)g0 * 4 + e];
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // keep those loads ahead of the weights
  issue(n < N ? n : N - 1, 0);   // a team past the last row loads it and never uses it
  __builtin_amdgcn_sched_barrier(0);
  float ss = 0.f;                                 // kNin: this thread's sum of h^2
  float rs = 1.f;                                 // kNin, factored: 1 / rms of h
  // exact: h and gamma wait in LDS (each thread's own entries) until the sum of
  // h^2 is known; factored: h * gamma staged at once
  uint4* const hs = xs + 4 * gc;
  uint4* const gs = xs + 8 * gc;
  auto stage_norm = [&](int e, uint4 r, uint4 dl, uint4 gw) {
    h8_t v = bits<h8_t>(r);
    if (ndel) v = v + bits<h8_t>(dl);
    if (nin.res_out && blockIdx.x == 0) reinterpret_cast<uint4*>(nin.res_out)[e] = bits<uint4>(v);
    const h8_t gm = bits<h8_t>(gw);
    h8_t o;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float f = (float)v[k];
      ss = __builtin_fmaf(f, f, ss);
      o[k] = (_Float16)(f * (float)gm[k]);
    }
    if (nin.exact) {
      gs[e] = gw;
      hs[e] = bits<uint4>(v);
    } else {
      xs[(e & 3) * gc + (e >> 2)] = pair_order(bits<uint4>(o));
    }
  };
  if constexpr (kNin) {
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      const int e = threadIdx.x + j * kBlock;
      if (e < 4 * gc) stage_norm(e, pr[j], pd[j], pg[j]);
    }
    for (int e = threadIdx.x + PRE * kBlock; e < 4 * gc; e += kBlock)
      stage_norm(e, nres[e], ndel ? ndel[e] : make_uint4(0u, 0u, 0u, 0u), ngam[e]);
    if (nin.exact) {
      const float r = rms_scale(block_sum<false>(ss, ssw), G * 32, nin.eps);   // ssw not reused
      for (int e = threadIdx.x; e < 4 * gc; e += kBlock) {
        const h8_t v = bits<h8_t>(hs[e]), gm = bits<h8_t>(gs[e]);
        h8_t o;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = norm_h(v[k], r, gm[k]);
        xs[(e & 3) * gc + (e >> 2)] = pair_order(bits<uint4>(o));
      }
    }
  } else {
    // unconditional, at the clamped index (a duplicate writes the same value), so
    // that the early loads stay where they are
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      int e = threadIdx.x + j * kBlock;
      e = e < 4 * gc ? e : 4 * gc - 1;
      xs[(e & 3) * gc + (e >> 2)] = pair_order(pr[j]);
    }
    for (int i = threadIdx.x + PRE * kBlock; i < 4 * gc; i += kBlock)
      xs[(i & 3) * gc + (i >> 2)] = pair_order(X[(int64_t)g0 * 4 + i]);
  }
  if (kNin && !nin.exact) {
    ss = team_sum<64>(ss);
    if ((threadIdx.x & 63) == 0) ssw[threadIdx.x >> 6] = ss;
  }
  float* const xsum = reinterpret_cast<float*>(xs + 4 * gc);   // kAffine: sum of x per group
  if constexpr (kAff) {
    auto group_sum = [&](const uint4 (&v4)[4]) {
      float t = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hw[4] = {v4[j].x, v4[j].y, v4[j].z, v4[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          t += half_to_float((uint16_t)(hw[i] & 0xFFFFu)) + half_to_float((uint16_t)(hw[i] >> 16));
      }
      return t;
    };
    // the first group from the early loads (a clamped duplicate writes the same sum)
    xsum[(int)threadIdx.x < gc ? (int)threadIdx.x : gc - 1] = group_sum(px);
    for (int g = threadIdx.x + kBlock; g < gc; g += kBlock) {
      uint4 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = X[(int64_t)(g0 + g) * 4 + j];
      xsum[g] = group_sum(v4);
    }
  }
  __syncthreads();
  if (kNin && !nin.exact) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) tot += ssw[w];
    rs = 1.f / __builtin_sqrtf(tot / (float)(G * 32) + nin.eps);
  }

  for (; n < N; n += nteams) {
    float acc[R];
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q] = 0.f;
    for (int t0 = 0; t0 < gc; t0 += LPR * UNR) {
      if (t0 > 0) issue(n, t0);
#pragma unroll
      for (int q = 0; q < R; ++q) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int graw = t0 + u * LPR + lane;
          const int g = graw < gc ? graw : gc - 1;
          const float p = group_dot(wv[q][u], xs, gc, g);
          const float sc = sval(sv[q][u]);
          float t = __builtin_fmaf(p, sc, acc[q]);
          if constexpr (kAff)
            t = __builtin_fmaf(__builtin_fmaf(7.f, sc, sval(bv[q][u])), xsum[g], t);
          acc[q] = graw < gc ? t : acc[q];
        }
      }
    }
    if (n + nteams < N) issue(n + nteams, 0);
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q] = team_sum<LPR>(acc[q]);
    if (lane == 0) {
      if constexpr (MODE == kGlu) {
        Y[n] = bits<uint16_t>(silu_mul_h((_Float16)acc[0], (_Float16)acc[1]));
      } else if constexpr (MODE == kGluNorm) {
        Y[n] = bits<uint16_t>(silu_mul_h((_Float16)(acc[0] * rs), (_Float16)(acc[1] * rs)));
      } else if constexpr (MODE == kPlainNorm) {
        Y[n] = float_to_half_rne(acc[0] * rs);
      } else if (splits == 1) {
        Y[n] = float_to_half_rne(acc[0]);
      } else {
        P[(int64_t)split * N + n] = acc[0];
      }
    }
  }
}

// ------------------------------------------------------------- M in 4..8 ---
// (2 and 3 rows run on the vector units, k_gemv_mx below.)  A workgroup stages X once and loops over tiles of 16 rows x one K slice (a
// workgroup per tile staged X once per 16 rows: at M = 8, K = 2048 that was 32 KB
// of X per 18 KB of weights); its four waves take interleaved chunks of four
// groups.  In a chunk, lane (c = lane/16, r = lane%16) loads group c of
// row r with one dwordx4; a 4x4 exchange among lanes r, r+16, r+32, r+48
// (permlane32/permlane16 swaps) leaves word c of every group of the chunk in lane
// (c, r), which is the B-operand layout of v_mfma_f32_16x16x32_f16 (column = row
// n, k block = c).  A = X rows (row m = r < M, zero above M), from LDS in the same
// pair order.  One MFMA per group into a fresh accumulator, then acc += s * D.
template <bool WIDE>
__global__ __launch_bounds__(kBlock) void k_gemv_mfma(const uint4* __restrict__ W,
                                                      const uint16_t* __restrict__ S,
                                                      const uint4* __restrict__ X,
                                                      uint16_t* __restrict__ Y,
                                                      float* __restrict__ P, int M, int N,
                                                      int G, int splits) {
  extern __shared__ uint4 xs[];   // [M][4*gc + 1]: row m, group g, word j at m*(4gc+1) + 4g + j
  __shared__ f4_t red[3][64];
  const int split = blockIdx.y;
  const int g0 = slice_begin(G, splits, split);
  const int gc = slice_begin(G, splits, split + 1) - g0;
  const int pitch = 4 * gc + 1;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, c = l >> 4, r = l & 15;
  const bool has_x = r < M;
  uint32_t* const stage = reinterpret_cast<uint32_t*>(xs + M * pitch) + wave * 512;
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const int nx = M * 4 * gc;
  auto x_at = [&](int i) {   // entry i of X's slice, row-major [M][4 gc]
    const int m = i / (4 * gc), rr = i - m * 4 * gc;
    return X[(int64_t)m * G * 4 + (int64_t)g0 * 4 + rr];
  };
  auto x_put = [&](int i, uint4 v) {
    const int m = i / (4 * gc), rr = i - m * 4 * gc;
    xs[m * pitch + rr] = pair_order(v);
  };

  if constexpr (WIDE) {
    // Blocks of eight groups ("chunks"): two loads of 8 rows x 128 contiguous bytes
    // (lane l: row 8h + l / 8, group l % 8; whole cache lines, where one group per
    // lane of 16 rows touches 16 half lines), through this wave's stage as word
    // planes [word][16 rows][8 groups], from which lane (c, r) reads word c of row
    // r's eight groups as 32 contiguous bytes; the row's eight scales in one load.
    // Wave w takes chunks 8w, 8w + 32, ... of every tile of 16 rows; every wave has
    // the same number per tile (CPW; a chunk past the slice is loaded from the
    // last one and not computed), so all four reach each tile's cross-wave sum
    // together.  The wave's chunks of all its workgroup's tiles form one sequence,
    // and the next chunk's loads are issued before a chunk is computed (two
    // register slots taken in turn).  X's first PX entries per thread and the first
    // chunk are loaded before X is staged, all without a branch, so the staging
    // waits for X only.
    const int CPW = (gc + 31) / 32;
    const int tstride = gridDim.x * 16;
    const int tiles = (N - (int)blockIdx.x * 16 + tstride - 1) / tstride;   // >= 1
    const int total = tiles * CPW;
    struct Chunk {
      uint4 raw[2];
      uint4 sv;
    };
    auto issue = [&](Chunk& C, int i) {
      i = i < total ? i : total - 1;         // past the end: the last chunk again, unused
      const int n0 = (int)blockIdx.x * 16 + (i / CPW) * tstride;
      int gb = 8 * wave + 32 * (i % CPW);
      gb = gb < gc ? gb : gc - 8;
      const int64_t rows_left = (int64_t)(N - n0);
      const uint4* wt = W + (int64_t)n0 * G + g0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = 8 * h + (l >> 3);
        C.raw[h] = load_nt(wt + (row < rows_left ? row : rows_left - 1) * G + gb + (l & 7));
      }
      const int n = n0 + r < N ? n0 + r : N - 1;
      C.sv = *reinterpret_cast<const uint4*>(S + (int64_t)n * G + g0 + gb);
    };
    constexpr int PX = 8;
    uint4 xp[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
      const int i = (int)threadIdx.x + j * kBlock;
      xp[j] = x_at(i < nx ? i : nx - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    Chunk A, B;
    issue(A, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PX; ++j) {   // a clamped duplicate writes the same value
      const int i = (int)threadIdx.x + j * kBlock;
      x_put(i < nx ? i : nx - 1, xp[j]);
    }
    for (int i = threadIdx.x + PX * kBlock; i < nx; i += kBlock) x_put(i, x_at(i));
    __syncthreads();

    f4_t acc = zero;
    auto consume = [&](const Chunk& C, int i) {
      const int ti = i / CPW, ci = i - ti * CPW;
      const int n0 = (int)blockIdx.x * 16 + ti * tstride;
      const int gb = 8 * wave + 32 * ci;
      if (gb < gc) {
        // the stage is read by other lanes of the wave: keep its writes and reads
        // in program order (a wave's LDS operations complete in order)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          stage[j * 128 + l] = (&C.raw[0].x)[j];
          stage[j * 128 + 64 + l] = (&C.raw[1].x)[j];
        }
        asm volatile("" ::: "memory");
        const uint4* sp = reinterpret_cast<const uint4*>(stage + c * 128 + r * 8);
        const uint4 wq0 = sp[0], wq1 = sp[1];
        asm volatile("" ::: "memory");
        const uint32_t wc[8] = {wq0.x, wq0.y, wq0.z, wq0.w, wq1.x, wq1.y, wq1.z, wq1.w};
        const uint32_t sw[4] = {C.sv.x, C.sv.y, C.sv.z, C.sv.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          h2_t q[4];
          dequant_word(wc[t], q);
          const h8_t Bq = {q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
          h8_t Ax = {};
          if (has_x) Ax = bits<h8_t>(xs[r * pitch + 4 * (gb + t) + c]);
          const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ax, Bq, zero, 0, 0, 0);
          const float sc = half_to_float((uint16_t)(sw[t >> 1] >> (16 * (t & 1))));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sc, d[e], acc[e]);
        }
      }
      if (ci == CPW - 1) {
        // the tile's end: add the four waves' partials in a fixed order
        if (wave > 0) red[wave - 1][l] = acc;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
          for (int w = 0; w < 3; ++w) acc += red[w][l];
          if (n0 + r < N) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 4 * c + e;
              if (m < M) {
                if (splits == 1)
                  Y[(int64_t)m * N + n0 + r] = float_to_half_rne(acc[e]);
                else
                  P[((int64_t)split * M + m) * N + n0 + r] = acc[e];
              }
            }
          }
        }
        __syncthreads();   // red is reused by the next tile
        acc = zero;
      }
    };
    for (int i = 0;; i += 2) {
      issue(B, i + 1);
      consume(A, i);
      if (i + 1 >= total) break;
      issue(A, i + 2);
      consume(B, i + 1);
      if (i + 2 >= total) break;
    }
    return;
  }

  for (int i = threadIdx.x; i < nx; i += kBlock) x_put(i, x_at(i));
  __syncthreads();
  // workgroups loop over tiles of 16 rows, so X is staged once per workgroup, not
  // once per tile
  for (int n0 = blockIdx.x * 16; n0 < N; n0 += gridDim.x * 16) {
    const int n = n0 + r < N ? n0 + r : N - 1;
    const uint4* wr = W + (int64_t)n * G + g0;
    const uint16_t* sr = S + (int64_t)n * G + g0;
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int gb = 4 * wave; gb < gc; gb += 16) {
      const int gl = gb + c < gc ? gb + c : gc - 1;
      const uint4 wv = load_nt(wr + gl);
      float s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = half_to_float(sr[gb + t < gc ? gb + t : gc - 1]);
      uint32_t v[4] = {wv.x, wv.y, wv.z, wv.w};
      transpose4(v);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int gt = gb + t < gc ? gb + t : gc - 1;
        h2_t q[4];
        dequant_word(v[t], q);
        const h8_t B = {q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
        h8_t A = {};
        if (has_x) A = bits<h8_t>(xs[r * pitch + 4 * gt + c]);
        const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, zero, 0, 0, 0);
        if (gb + t < gc) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(s[t], d[e], acc[e]);
        }
      }
    }
    // add the four waves' partials in a fixed order
    if (wave > 0) red[wave - 1][l] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w) acc += red[w][l];
      if (n0 + r < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * c + e;
          if (m < M) {
            if (splits == 1)
              Y[(int64_t)m * N + n0 + r] = float_to_half_rne(acc[e]);
            else
              P[((int64_t)split * M + m) * N + n0 + r] = acc[e];
          }
        }
      }
    }
    __syncthreads();   // red is reused by the next tile
  }
}

// ------------------------------------------------------------- M in 2..3 ---
// The M = 1 kernel's layout with XM rows of x: a team of LPR lanes per row, lane i
// taking groups i, i + LPR, ... of the slice (one trip: the launch picks UNR so
// that a lane's groups fit it), X staged as XM sets of the M = 1 kernel's
// pair-ordered planes.  Each group's words are decoded once (the exact q - 7
// pairs) and dotted with every row of X, each row with the M = 1 kernel's own
// chains, so a row's output equals the M = 1 GEMV of that row when both run as
// one slice.  Up to three rows this beats the 16-row MFMA tile, which leaves most
// of its A operand empty (151936 x 2048: 47 -> 43 us at M = 2; 12288 x 2048: 9.6 ->
// 8.8 us at M = 3); at four, X's LDS reads cost more than the MFMA saves.
template <int LPR, int UNR, int XM>
__global__ __launch_bounds__(kBlock) void k_gemv_mx(const uint4* __restrict__ W,
                                                    const uint16_t* __restrict__ S,
                                                    const uint4* __restrict__ X,
                                                    uint16_t* __restrict__ Y,
                                                    float* __restrict__ P, int N, int G,
                                                    int splits) {
  extern __shared__ uint4 xs[];   // [XM][4][gc]
  const int split = blockIdx.y;
  const int g0 = slice_begin(G, splits, split);
  const int gc = slice_begin(G, splits, split + 1) - g0;
  const int lane = threadIdx.x & (LPR - 1);
  const int team = (int)((blockIdx.x * (unsigned)kBlock + threadIdx.x) / LPR);
  const int nteams = (int)(gridDim.x * (unsigned)(kBlock / LPR));
  uint4 wv[UNR];
  uint16_t sv[UNR];
  auto issue = [&](int n, int t0) {
    const uint4* wr = W + (int64_t)n * G + g0;
    const uint16_t* sr = S + (int64_t)n * G + g0;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      int g = t0 + u * LPR + lane;
      g = g < gc ? g : gc - 1;
      wv[u] = load_nt(wr + g);
      sv[u] = sr[g];
    }
  };
  // entry e of X's slice, row-major [XM][4 gc]: block r of row m
  const int nx = XM * 4 * gc;
  auto x_at = [&](int e) {
    const int m = e / (4 * gc), r = e - m * 4 * gc;
    return X[(int64_t)m * G * 4 + (int64_t)g0 * 4 + r];
  };
  auto x_put = [&](int e, uint4 v) {
    const int m = e / (4 * gc), r = e - m * 4 * gc;
    xs[m * 4 * gc + (r & 3) * gc + (r >> 2)] = pair_order(v);
  };
  // this thread's first PRE entries are loaded before the weights, without a
  // branch, so that the staging waits for them only (as in the M = 1 kernel)
  constexpr int PRE = 4;
  uint4 pr[PRE];
#pragma unroll
  for (int j = 0; j < PRE; ++j) {
    const int e = (int)threadIdx.x + j * kBlock;
    pr[j] = x_at(e < nx ? e : nx - 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  int n = team;
  issue(n < N ? n : N - 1, 0);   // a team past the last row loads it and never uses it
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < PRE; ++j) {   // a clamped duplicate writes the same value
    const int e = (int)threadIdx.x + j * kBlock;
    x_put(e < nx ? e : nx - 1, pr[j]);
  }
  for (int e = threadIdx.x + PRE * kBlock; e < nx; e += kBlock) x_put(e, x_at(e));
  __syncthreads();

  for (; n < N; n += nteams) {
    float acc[XM];
#pragma unroll
    for (int m = 0; m < XM; ++m) acc[m] = 0.f;
    for (int t0 = 0; t0 < gc; t0 += LPR * UNR) {
      if (t0 > 0) issue(n, t0);
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int graw = t0 + u * LPR + lane;
        const int g = graw < gc ? graw : gc - 1;
        const uint32_t wj[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
        h2_t q[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dequant_word(wj[j], q[j]);
        const float sc = half_to_float(sv[u]);
#pragma unroll
        for (int m = 0; m < XM; ++m) {
          const uint4* xm = xs + m * 4 * gc;
          float a = 0.f, b = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint4 xv = xm[j * gc + g];
            a = __builtin_amdgcn_fdot2(q[j][0], bits<h2_t>(xv.x), a, false);
            b = __builtin_amdgcn_fdot2(q[j][1], bits<h2_t>(xv.y), b, false);
            a = __builtin_amdgcn_fdot2(q[j][2], bits<h2_t>(xv.z), a, false);
            b = __builtin_amdgcn_fdot2(q[j][3], bits<h2_t>(xv.w), b, false);
          }
          const float t = __builtin_fmaf(a + b, sc, acc[m]);
          acc[m] = graw < gc ? t : acc[m];
        }
      }
    }
    if (n + nteams < N) issue(n + nteams, 0);
#pragma unroll
    for (int m = 0; m < XM; ++m) acc[m] = team_sum<LPR>(acc[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < XM; ++m) {
        if (splits == 1)
          Y[(int64_t)m * N + n] = float_to_half_rne(acc[m]);
        else
          P[((int64_t)split * XM + m) * N + n] = acc[m];
      }
    }
  }
}

// Second pass of split-K: out[i] = fp16(sum over s ascending of P[s*count + i]).
__global__ __launch_bounds__(kBlock) void k_combine(const float* __restrict__ P,
                                                    uint16_t* __restrict__ Y, int64_t count,
                                                    int splits) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < count; i += stride) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += P[(int64_t)s * count + i];
    Y[i] = float_to_half_rne(acc);
  }
}

// Dynamic LDS above 64 KB must be allowed per kernel (gfx950 has 160 KB per CU).
template <typename F>
hipError_t allow_lds(F* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

int pow2_floor(int64_t v) {
  int p = 1;
  while ((int64_t)p * 2 <= v) p *= 2;
  return p;
}

int choose_lpr(int64_t G) {
  int l = pow2_floor(G / 3 > 0 ? G / 3 : 1);
  return l < 4 ? 4 : (l > 64 ? 64 : l);
}

// a.N: the outputs (kGlu: half the matrix's rows)
template <int LPR, int UNR, int MODE>
hipError_t launch_m1_unr(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                         hipStream_t s, const uint16_t* biases, const NormIn& nin) {
  const int64_t G = a.K / 32;
  const int64_t teams_per_block = kBlock / LPR;
  int64_t blocks = (a.N + teams_per_block - 1) / teams_per_block;
  // Eight workgroups per compute unit, each looping over its share of the rows:
  // every workgroup stages x once, so a grid of one workgroup per 8 rows re-reads
  // it 6 KB per 14 KB of weights (K = 3072); measured best against 2, 4, 16, 64.
  // The folded-norm modes stage from three vectors (residual, delta, gamma), and
  // take three per unit (Phi-3-shaped token loop, exact norms: 0.847 ms at 2,
  // 0.828 at 3, 0.860 at 4).
  constexpr bool kNin = MODE == kPlainNorm || MODE == kGluNorm;
  const int64_t cap = (int64_t)d.cus * (kNin ? 3 : 8);
  if (blocks > cap) blocks = cap;
  const int64_t gmax = (G + p.splits - 1) / p.splits;
  const size_t lds =
      (size_t)gmax * (MODE == kAffine || MODE == kAffineB ? 68 : kNin && nin.exact ? 192 : 64);
  const dim3 grid((unsigned)blocks, (unsigned)p.splits);
  if (hipError_t e = allow_lds(k_gemv_m1<LPR, UNR, MODE>, lds)) return e;
  hipLaunchKernelGGL((k_gemv_m1<LPR, UNR, MODE>), grid, dim3(kBlock), lds, s,
                     reinterpret_cast<const uint4*>(a.words), a.scales, biases,
                     reinterpret_cast<const uint4*>(a.x), a.y, part, (int)a.N, (int)G, p.splits,
                     nin);
  return hipGetLastError();
}

// groups per lane per trip: the whole slice in one trip up to 8 (larger slices,
// from an explicit split count, take several trips), with no group beyond the
// slice up to 6: a lane's groups past the slice are loaded and computed before
// being discarded, and K = 3072 (96 groups, 32 lanes) at 4 per lane spent a
// quarter of every lane's work there (262144 x 3072: 91.9 -> 72.1 us at 3)
template <int LPR, int MODE>
hipError_t launch_m1(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                     hipStream_t s, const uint16_t* biases, const NormIn& nin) {
  const int64_t G = a.K / 32;
  const int64_t per_lane = ((G + p.splits - 1) / p.splits + LPR - 1) / LPR;
  switch (per_lane) {
    case 0: case 1: case 2: return launch_m1_unr<LPR, 2, MODE>(a, p, part, d, s, biases, nin);
    case 3: return launch_m1_unr<LPR, 3, MODE>(a, p, part, d, s, biases, nin);
    case 4: return launch_m1_unr<LPR, 4, MODE>(a, p, part, d, s, biases, nin);
    case 5: return launch_m1_unr<LPR, 5, MODE>(a, p, part, d, s, biases, nin);
    case 6: return launch_m1_unr<LPR, 6, MODE>(a, p, part, d, s, biases, nin);
    default: return launch_m1_unr<LPR, 8, MODE>(a, p, part, d, s, biases, nin);
  }
}

// biases: kAffine only; nin: kPlainNorm and kGluNorm only
template <int MODE>
hipError_t launch_m1_lpr(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                         hipStream_t s, const uint16_t* biases = nullptr,
                         const NormIn& nin = NormIn{}) {
  switch (p.lanes_per_row) {
    case 4: return launch_m1<4, MODE>(a, p, part, d, s, biases, nin);
    case 8: return launch_m1<8, MODE>(a, p, part, d, s, biases, nin);
    case 16: return launch_m1<16, MODE>(a, p, part, d, s, biases, nin);
    case 32: return launch_m1<32, MODE>(a, p, part, d, s, biases, nin);
    default: return launch_m1<64, MODE>(a, p, part, d, s, biases, nin);
  }
}

template <int LPR, int UNR, int XM>
hipError_t launch_mx_unr(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                         hipStream_t s) {
  const int64_t G = a.K / 32;
  const int64_t gmax = (G + p.splits - 1) / p.splits;
  const size_t lds = (size_t)XM * gmax * 64;
  int64_t blocks = (a.N + kBlock / LPR - 1) / (kBlock / LPR);
  // workgroups loop over their rows: at most eight per compute unit, fewer when
  // the LDS of X allows fewer at once
  int64_t per_cu = (int64_t)(d.lds_per_block / (lds > 0 ? lds : 1));
  per_cu = per_cu < 1 ? 1 : per_cu > 8 ? 8 : per_cu;
  if (blocks > (int64_t)d.cus * per_cu) blocks = (int64_t)d.cus * per_cu;
  const dim3 grid((unsigned)blocks, (unsigned)p.splits);
  if (hipError_t e = allow_lds(k_gemv_mx<LPR, UNR, XM>, lds)) return e;
  hipLaunchKernelGGL((k_gemv_mx<LPR, UNR, XM>), grid, dim3(kBlock), lds, s,
                     reinterpret_cast<const uint4*>(a.words), a.scales,
                     reinterpret_cast<const uint4*>(a.x), a.y, part, (int)a.N, (int)G, p.splits);
  return hipGetLastError();
}

template <int LPR, int XM>
hipError_t launch_mx(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                     hipStream_t s) {
  const int64_t G = a.K / 32;
  const int64_t per_lane = ((G + p.splits - 1) / p.splits + LPR - 1) / LPR;
  switch (per_lane) {
    case 0: case 1: case 2: return launch_mx_unr<LPR, 2, XM>(a, p, part, d, s);
    case 3: return launch_mx_unr<LPR, 3, XM>(a, p, part, d, s);
    case 4: return launch_mx_unr<LPR, 4, XM>(a, p, part, d, s);
    case 5: return launch_mx_unr<LPR, 5, XM>(a, p, part, d, s);
    case 6: return launch_mx_unr<LPR, 6, XM>(a, p, part, d, s);
    default: return launch_mx_unr<LPR, 8, XM>(a, p, part, d, s);
  }
}

template <int XM>
hipError_t launch_mx_lpr(const GemvArgs& a, const GemvPlan& p, float* part, const DeviceInfo& d,
                         hipStream_t s) {
  switch (p.lanes_per_row) {
    case 4: return launch_mx<4, XM>(a, p, part, d, s);
    case 8: return launch_mx<8, XM>(a, p, part, d, s);
    case 16: return launch_mx<16, XM>(a, p, part, d, s);
    case 32: return launch_mx<32, XM>(a, p, part, d, s);
    default: return launch_mx<64, XM>(a, p, part, d, s);
  }
}

}  // namespace

int64_t max_groups_per_slice(const DeviceInfo& d, int64_t M) {
  // M <= kMxMax (k_gemv_m1, k_gemv_mx): 64 bytes of LDS per group and row.  More: M
  // rows of (4 g + 1) uint4 plus 3 KB of cross-wave partials and 2 KB of stage per wave.
  const int64_t lds = (int64_t)d.lds_per_block;
  if (M <= kMxMax) return lds / (64 * (M < 1 ? 1 : M));
  return ((lds - 3 * 64 * 16 - (kBlock / 64) * 2048) / (16 * M) - 1) / 4;
}

GemvPlan plan_splits(const DeviceInfo& d, int64_t M, int64_t N, int64_t K, int splits) {
  GemvPlan p;
  p.splits = splits;
  p.lanes_per_row = M <= kMxMax ? choose_lpr(K / 32) : 64;
  p.ws_bytes = splits > 1 ? (size_t)4 * splits * M * N : 0;
  (void)d;
  return p;
}

GemvPlan plan_auto(const DeviceInfo& d, int64_t M, int64_t N, int64_t K) {
  const int64_t G = K / 32;
  const int64_t gmax = max_groups_per_slice(d, M);
  int64_t splits = (G + gmax - 1) / gmax;       // fit the slice of x in LDS
  int64_t blocks;
  if (M <= kMxMax) {
    const int lpr = choose_lpr(G);
    blocks = (N + kBlock / lpr - 1) / (kBlock / lpr);
  } else {
    blocks = (N + 15) / 16;
  }
  // too few workgroups to give every compute unit one: split K as well (a
  // workgroup's loads are all in flight at once, so one per unit already
  // streams; a second split-K pass costs more than the rows it would add)
  const int64_t want = M <= kMxMax ? (int64_t)d.cus : 2 * (int64_t)d.cus;
  if (blocks * splits < want) {
    int64_t s2 = (want + blocks - 1) / blocks;
    const int64_t smax = M <= kMxMax ? G / 8 : G / 16;
    if (s2 > smax) s2 = smax;
    if (s2 > splits) splits = s2;
  }
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  return plan_splits(d, M, N, K, (int)splits);
}

hipError_t launch_gemv(const DeviceInfo& d, const GemvArgs& a, const GemvPlan& p, void* ws,
                       hipStream_t s) {
  float* part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
  uint16_t* out = a.y;
  hipError_t e;
  if (a.M == 1) {
    e = launch_m1_lpr<kPlain>(a, p, part, d, s);
  } else if (a.M <= kMxMax) {
    e = a.M == 2 ? launch_mx_lpr<2>(a, p, part, d, s) : launch_mx_lpr<3>(a, p, part, d, s);
  } else {
    const int64_t G = a.K / 32;
    const int64_t gmax = (G + p.splits - 1) / p.splits;
    const size_t lds = (size_t)a.M * (4 * gmax + 1) * 16 + (kBlock / 64) * 2048;
    // as many workgroups as fit the device at once (LDS bounds them: X is M rows
    // of the slice), each looping over tiles
    int64_t tiles = (a.N + 15) / 16;
    const int64_t per_cu = lds > 0 ? (int64_t)(d.lds_per_block / (lds + 3 * 64 * 16)) : 8;
    const int64_t cap = (int64_t)d.cus * (per_cu < 1 ? 1 : per_cu > 8 ? 8 : per_cu);
    if (tiles * p.splits > cap) tiles = (cap + p.splits - 1) / p.splits;
    const dim3 grid((unsigned)tiles, (unsigned)p.splits);
    // the eight-group chunks need whole chunks in every slice and 16-byte aligned
    // scale runs
    bool wide = G % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15u) == 0;
    for (int sp = 0; wide && sp < p.splits; ++sp)
      wide = slice_begin((int)G, p.splits, sp) % 8 == 0 &&
             slice_begin((int)G, p.splits, sp + 1) % 8 == 0;
    auto kern = wide ? k_gemv_mfma<true> : k_gemv_mfma<false>;
    if (hipError_t e2 = allow_lds(kern, lds)) return e2;
    hipLaunchKernelGGL(kern, grid, dim3(kBlock), lds, s,
                       reinterpret_cast<const uint4*>(a.words), a.scales,
                       reinterpret_cast<const uint4*>(a.x), out, part, (int)a.M, (int)a.N,
                       (int)G, p.splits);
    e = hipGetLastError();
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t count = a.M * a.N;
  int64_t blocks = (count + kBlock - 1) / kBlock;
  if (blocks > (int64_t)d.cus * 8) blocks = (int64_t)d.cus * 8;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(kBlock), 0, s, part, out, count,
                     p.splits);
  return hipGetLastError();
}

hipError_t launch_gemv_affine(const DeviceInfo& d, const uint32_t* W, const uint16_t* S,
                              const uint16_t* B, const uint16_t* X, uint16_t* Y, int64_t N,
                              int64_t K, bool bf16, hipStream_t s) {
  const GemvArgs a{W, S, X, Y, 1, N, K};
  const GemvPlan p = plan_splits(d, 1, N, K, 1);
  if ((size_t)(K / 32) * 68 > d.lds_per_block) return hipErrorInvalidValue;
  return bf16 ? launch_m1_lpr<kAffineB>(a, p, nullptr, d, s, B)
              : launch_m1_lpr<kAffine>(a, p, nullptr, d, s, B);
}

hipError_t launch_gemv_norm_in(const DeviceInfo& d, const uint32_t* words,
                               const uint16_t* scales, const NormIn& nin, uint16_t* y,
                               int64_t N, int64_t K, bool glu, hipStream_t s) {
  if (!nin.res_in || !nin.gamma || (size_t)(K / 32) * (nin.exact ? 192 : 64) > d.lds_per_block)
    return hipErrorInvalidValue;
  const GemvArgs a{words, scales, nullptr, y, 1, N, K};
  const GemvPlan p = plan_splits(d, 1, glu ? 2 * N : N, K, 1);
  return glu ? launch_m1_lpr<kGluNorm>(a, p, nullptr, d, s, nullptr, nin)
             : launch_m1_lpr<kPlainNorm>(a, p, nullptr, d, s, nullptr, nin);
}

hipError_t launch_gemv_glu(const DeviceInfo& d, const uint32_t* words, const uint16_t* scales,
                           const uint16_t* x, uint16_t* h, int64_t F, int64_t K,
                           const GemvPlan& p, hipStream_t s) {
  if (p.splits != 1) return hipErrorInvalidValue;
  const GemvArgs a{words, scales, x, h, 1, F, K};
  return launch_m1_lpr<kGlu>(a, p, nullptr, d, s);
}

}  // namespace q4
