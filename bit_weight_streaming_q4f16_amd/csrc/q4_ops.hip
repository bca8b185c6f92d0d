// The steps of the decode loop around its GEMVs (Zero TVM documentation, "Decode
// loop"): the token's embedding row from a q4f16_1 table, RMSNorm, the residual
// add fused with RMSNorm ("addNorm"), and the argmax over the LM head's logits.
// Each is one small kernel, one workgroup per row; they move a few KB each, so
// what they cost is their launch and one memory round trip.
#include "q4_internal.h"
#include "q4_device.h"

namespace q4 {
namespace {

// One thread per 32-weight group of the chosen row: (q - 7) * s is exact in fp32
// (a 4-bit integer times an fp16), so each output is rounded once.
__global__ __launch_bounds__(kBlock) void k_embed_rows(const uint4* __restrict__ words,
                                                       const uint16_t* __restrict__ scales,
                                                       int64_t N, int G,
                                                       const int32_t* __restrict__ tokens,
                                                       uint4* __restrict__ out,
                                                       const int32_t* __restrict__ seq,
                                                       const int32_t* __restrict__ counter) {
  const int m = blockIdx.y;
  const int g = blockIdx.x * kBlock + threadIdx.x;
  if (g >= G) return;
  const int64_t t = counter ? seq[counter[0]] : tokens[m];
  uint4* o = out + ((int64_t)m * G + g) * 4;
  if (t < 0 || t >= N) {
    const uint4 nan4 = make_uint4(0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = nan4;
    return;
  }
  const uint4 w = words[t * G + g];
  const float s = (float)bits<_Float16>(scales[t * G + g]);
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h8_t h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)((float)((int)((wv[j] >> (4 * i)) & 0xFu) - 7) * s);
    o[j] = bits<uint4>(h);
  }
}

// RMSNorm of one row per workgroup, blocks of 8 halves, in the pieces of
// q4_internal.h (the GEMVs that fold the norm in stage the same bits); with
// `delta`, the row is first res_out = fp16(res_in + delta) (a native fp16 add:
// rounded once).  The second pass re-reads what this thread read or wrote in the
// first.
__global__ __launch_bounds__(kBlock) void k_rmsnorm(const uint4* __restrict__ delta,
                                                    const uint4* res_in,
                                                    const uint4* __restrict__ gamma, float eps,
                                                    int blocks, uint4* res_out,
                                                    uint4* __restrict__ out) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint4* x = res_in + row * blocks;
  uint4* r = res_out ? res_out + row * blocks : nullptr;
  float ss = 0.f;
  for (int b = threadIdx.x; b < blocks; b += kBlock) {
    h8_t v = bits<h8_t>(x[b]);
    if (delta) {
      v = v + bits<h8_t>(delta[row * blocks + b]);
      r[b] = bits<uint4>(v);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = (float)v[i];
      ss = __builtin_fmaf(f, f, ss);
    }
  }
  const float tot = block_sum(ss, red);
  const float rs = rms_scale(tot, blocks * 8, eps);
  const uint4* src = delta ? r : x;
  for (int b = threadIdx.x; b < blocks; b += kBlock) {
    const h8_t v = bits<h8_t>(src[b]), g = bits<h8_t>(gamma[b]);
    h8_t o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = norm_h(v[i], rs, g[i]);
    out[row * blocks + b] = bits<uint4>(o);
  }
}

// Largest value of a row, ties to the lowest index, NaN skipped (none: 0).  One
// workgroup of kArgThreads per row; a 16-byte aligned row is read as chunks of 8
// values, four chunks per thread in flight (a row of the LM head's 32064 logits is
// then one or two memory round trips, not a hundred dependent loads).  Within a
// thread values are seen in increasing index order and only a larger value
// replaces the best, so ties keep the lowest index; across threads the merge
// compares indices.
constexpr int kArgThreads = 1024;
__global__ __launch_bounds__(kArgThreads) void k_argmax(const uint16_t* __restrict__ x,
                                                        int64_t N, int32_t* __restrict__ out,
                                                        int32_t* __restrict__ seq,
                                                        int32_t* __restrict__ counter) {
  __shared__ float sv[kArgThreads / 64];
  __shared__ int64_t si[kArgThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * N;
  float bv = 0.f;
  int64_t bi = -1;
  auto see = [&](float v, int64_t n) {
    if (v == v && (bi < 0 || v > bv)) {
      bv = v;
      bi = n;
    }
  };
  int64_t head = 0;
  if ((reinterpret_cast<uintptr_t>(xr) & 15u) == 0) {
    const int64_t nch = N / 8;
    const uint4* xv = reinterpret_cast<const uint4*>(xr);
    for (int64_t c0 = threadIdx.x; c0 < nch; c0 += 4 * kArgThreads) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + (int64_t)u * kArgThreads;
        w[u] = c < nch ? xv[c] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + (int64_t)u * kArgThreads;
        if (c < nch) {
          const h8_t h = bits<h8_t>(w[u]);
#pragma unroll
          for (int e = 0; e < 8; ++e) see((float)h[e], c * 8 + e);
        }
      }
    }
    head = nch * 8;
  }
  for (int64_t n = head + threadIdx.x; n < N; n += kArgThreads)
    see((float)bits<_Float16>(xr[n]), n);
  // better: a value (bi >= 0) that is larger, or equal with a lower index
  auto take = [](float& v, int64_t& i, float ov, int64_t oi) {
    if (oi >= 0 && (i < 0 || ov > v || (ov == v && oi < i))) {
      v = ov;
      i = oi;
    }
  };
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int64_t oi = __shfl_xor(bi, o, 64);
    take(bv, bi, ov, oi);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = sv[0];
    int64_t i = si[0];
    for (int w = 1; w < kArgThreads / 64; ++w) take(v, i, sv[w], si[w]);
    const int32_t tok = (int32_t)(i < 0 ? 0 : i);
    out[row] = tok;
    if (counter) {   // a multi-step decode: the next step's token, one grid of one row
      const int32_t c = counter[0];
      seq[c + 1] = tok;
      counter[0] = c + 1;
    }
  }
}

__global__ void k_counter_reset(int32_t* counter) { counter[0] = 0; }

}  // namespace

hipError_t launch_counter_reset(int32_t* counter, hipStream_t s) {
  hipLaunchKernelGGL(k_counter_reset, dim3(1), dim3(1), 0, s, counter);
  return hipGetLastError();
}

hipError_t launch_embed_rows(const uint32_t* words, const uint16_t* scales, int64_t N, int64_t K,
                             const int32_t* tokens, int64_t M, uint16_t* out, hipStream_t s,
                             const int32_t* seq, const int32_t* counter) {
  if (counter && M != 1) return hipErrorInvalidValue;
  const int G = (int)(K / 32);
  hipLaunchKernelGGL(k_embed_rows, dim3((G + kBlock - 1) / kBlock, (unsigned)M), dim3(kBlock), 0,
                     s, reinterpret_cast<const uint4*>(words), scales, N, G, tokens,
                     reinterpret_cast<uint4*>(out), seq, counter);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* delta, const uint16_t* res_in, const uint16_t* gamma,
                          float eps, int64_t M, int64_t K, uint16_t* res_out, uint16_t* out,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)M), dim3(kBlock), 0, s,
                     reinterpret_cast<const uint4*>(delta), reinterpret_cast<const uint4*>(res_in),
                     reinterpret_cast<const uint4*>(gamma), eps, (int)(K / 8),
                     reinterpret_cast<uint4*>(res_out), reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_argmax(const uint16_t* x, int64_t M, int64_t N, int32_t* out, hipStream_t s,
                         int32_t* seq, int32_t* counter) {
  if (counter && M != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_argmax, dim3((unsigned)M), dim3(kArgThreads), 0, s, x, N, out, seq,
                     counter);
  return hipGetLastError();
}

}  // namespace q4
