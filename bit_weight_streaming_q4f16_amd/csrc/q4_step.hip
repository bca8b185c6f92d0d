// Persistent decode-step kernel: every M = 1 GEMV of a layer list in ONE launch.
//
// The Zero TVM decode loop runs the projections of every layer and then the LM
// head ("Decode loop"); decode is bandwidth-bound, so what matters is that the
// weight stream never stops (everything-webgpu AI.md: time per token scales with
// weight bytes; the launches themselves are a separate cost term).  Separate
// kernels per GEMV stop the stream at every boundary: the next kernel cannot
// issue a load before the previous one drains, and each small GEMV pays a fixed
// latency chain (stage x, first load round trip, reduction, drain).  Here the
// weights of later GEMVs are already in flight while earlier ones finish,
// because weights never depend on activations.
//
// One workgroup of 16 waves per compute unit (cooperative launch: all resident):
//  * 12 compute waves: a workgroup's items -- row-steps of every GEMV, in list
//    order -- are claimed from an LDS counter, B at a time, by whichever wave
//    is ready for more.  A wave works in bursts of B = 2 items:
//    it issues all loads of a burst (per item and lane, 4 x dwordx4 of packed
//    words and 4 fp16 scales), then consumes them, so the loads of the next
//    burst overlap this burst's arithmetic on the other waves.  An item is one
//    row per team of 2^lpr lanes, each lane holding up to 4 groups, so rows up
//    to K = 8192.  Results go to an LDS y buffer: these waves never wait on a
//    global store (on gfx9 stores and loads share one in-order counter).
//  * 4 sync waves, each owning every 4th GEMV: stage x of the GEMV into one of
//    8 LDS buffers (pair-ordered, with per-group offset terms) once the GEMVs it
//    depends on are complete on every workgroup, copy finished y rows from LDS
//    to memory, and publish per-GEMV completion with an agent-scope atomic that
//    other workgroups poll.  Their waits never hold back the weight stream.
//
// Dependencies (decided on the host): descriptor k waits for descriptor dep[k]
// (and, by list order, everything before it) to complete on all workgroups
// before its x is read.  Default: only where an earlier descriptor writes memory
// that k reads or writes; the "ordered" mode makes every descriptor wait for its
// predecessor, as in a decode step whose GEMVs feed each other.
#include <algorithm>
#include <climits>
#include <cstring>

#include "q4f16.h"
#include "q4_step.h"
#include "q4_device.h"

namespace q4 {
namespace {

template <typename T>
__device__ __forceinline__ const Q4_GLOBAL T* gptr(const T* p) {
  return (const Q4_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ Q4_GLOBAL T* gptr_mut(T* p) {
  return (Q4_GLOBAL T*)p;
}

// The fields of a descriptor a compute wave needs, read with scalar loads issued
// as inline assembly.  Read as ordinary loads, they become vector loads (the
// compiler cannot prove the table unchanged across the kernel's own stores), and
// using one would first drain every weight load the wave has in flight
// (vmcnt(0)) -- at every GEMV boundary, in the middle of a burst.
struct CursorDesc {
  const Q4_GLOBAL uint4* W;
  const Q4_GLOBAL uint16_t* S;
  int N, G, lg, C, steps, flags, sbase, srem;
};
__device__ __forceinline__ CursorDesc read_desc(const StepDesc* d) {
  u32x4_g ws;
  u32x8_s rest;        // N, G, lpr_log2 | C << 16, steps, dep, flags, sbase, srem
  asm volatile(
      "s_load_dwordx4 %0, %2, 0x0\n\t"
      "s_load_dwordx8 %1, %2, 0x20\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(ws), "=&s"(rest)
      : "s"(d));
  static_assert(offsetof(StepDesc, S) == 8 && offsetof(StepDesc, N) == 32 &&
                    offsetof(StepDesc, G) == 36 && offsetof(StepDesc, lpr_log2) == 40 &&
                    offsetof(StepDesc, C) == 42 && offsetof(StepDesc, steps) == 44 &&
                    offsetof(StepDesc, flags) == 52 && offsetof(StepDesc, sbase) == 56 &&
                    offsetof(StepDesc, srem) == 60,
                "descriptor offsets read by the compute waves");
  CursorDesc r;
  r.W = (const Q4_GLOBAL uint4*)(((uint64_t)ws[1] << 32) | ws[0]);
  r.S = (const Q4_GLOBAL uint16_t*)(((uint64_t)ws[3] << 32) | ws[2]);
  r.N = (int)rest[0];
  r.G = (int)rest[1];
  r.lg = (int)(rest[2] & 0xFFFFu);
  r.C = (int)(rest[2] >> 16);
  r.steps = (int)rest[3];
  r.flags = (int)rest[5];
  r.sbase = (int)rest[6];
  r.srem = (int)rest[7];
  return r;
}


// An affine GEMV's bias pointer, read the same way (at GEMV transitions only).
__device__ __forceinline__ const Q4_GLOBAL uint16_t* read_bias(const StepDesc* d) {
  u32x2_g b;
  asm volatile(
      "s_load_dwordx2 %0, %1, 0x48\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(b)
      : "s"(d));
  static_assert(offsetof(StepDesc, Bs) == 72, "bias pointer offset read by the compute waves");
  return (const Q4_GLOBAL uint16_t*)(((uint64_t)b[1] << 32) | b[0]);
}

// An affine scale or bias (bf16, or fp16 with kAffineF16) as fp32, exactly.
__device__ __forceinline__ float affine_value(uint16_t h, bool f16) {
  return f16 ? (float)bits<_Float16>(h) : bits<float>((uint32_t)h << 16);
}

// An affine pair's scale and bias from the two lanes that loaded them (the even
// lane the scale, the odd lane the bias; neighbours in a row's team).  Every lane
// of the wave must be active.
__device__ __forceinline__ void pair_values(uint16_t own, bool f16, float& sc, float& bi) {
  const uint16_t other = (uint16_t)bits<uint32_t>(dpp<0xB1>(bits<float>((uint32_t)own)));
  const bool odd = (threadIdx.x & 1) != 0;
  sc = affine_value(odd ? other : own, f16);
  bi = affine_value(odd ? own : other, f16);
}

constexpr int kWaves = kStepThreads / 64;   // 16
constexpr int kSync = 4;                    // sync waves (stage x, copy out y)
constexpr int kCompute = kWaves - kSync;    // compute waves
static_assert(kXBufs % kSync == 0, "a GEMV and the one whose x buffer it reuses share an owner");
constexpr unsigned kSpinLimit = 1u << 24;   // bounded waits (about a second)
constexpr unsigned kTagSpinLimit = 1u << 18; // polls of tagged pairs (a memory round trip each)

struct Shared {
  int x_ready[kXBufs];   // GEMV index whose x sits in buffer b (-1: none yet)
  int local_done[kXBufs];// compute-wave completions per buffer (monotonic)
  int err;               // a compute wave's wait ran out (copied out by the sync wave)
  int next_item;         // next unclaimed item of this workgroup's sequence
};

// First row-step of workgroup wg (the even split of the descriptor's row-steps
// computed on the host; wg == grid size gives the end).
__device__ __forceinline__ int wg_step(int sbase, int srem, int wg) {
  return wg * sbase + (wg < srem ? wg : srem);
}

// LDS layout, per x buffer b (kXBufs of them):
//   xbuf[b]: 4 planes of maxG pair-ordered blocks (uint4); maxG is the largest
//            padded group count (lanes per row x groups per lane) of the list,
//            blocks past a GEMV's own G are zero
//   cbuf[b]: maxG floats, the offset term of each group (zero past G)
//   ybuf[b]: ybuf_rows fp16 results of this workgroup's rows
//   sbuf[b]: (AFF) maxG floats, 2^-20 times each group's sum of x (affine GEMVs)
// AFF: the list holds affine GEMVs (kAffine): every item also loads its biases
// (from an empty resource for the other formats), so the load count per item stays
// fixed; lists without them take the variant that never issues those loads.
template <int B, int NX, bool AFF>
__global__ __launch_bounds__(kStepThreads) void k_step(const StepDesc* __restrict__ D, int n,
                                                       unsigned* __restrict__ ctl, int maxG,
                                                       int ybuf_rows,
                                                       const int4* __restrict__ ranges) {
  static_assert(NX <= kXBufs && NX % kSync == 0, "x buffers");
  unsigned* const done = ctl + kCtlWords;       // completion counters
  // this launch's hand-over epoch: one past the last launch's (never 0); the
  // last workgroup to finish stores it for the next launch
  unsigned epoch = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  epoch = epoch + 1u == 0u ? 1u : epoch + 1u;
  extern __shared__ uint4 smem[];
  __shared__ Shared sh;
  uint4* xbuf = smem;                                                           // [NX][4][maxG]
  float* cbuf = reinterpret_cast<float*>(smem + NX * 4 * maxG);                 // [NX][maxG]
  uint16_t* ybuf = reinterpret_cast<uint16_t*>(cbuf + NX * maxG);              // [NX][rows]
  float* sbuf = reinterpret_cast<float*>(ybuf + NX * ybuf_rows);                // AFF: [NX][maxG]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x, nwg = gridDim.x;
  if (threadIdx.x < kXBufs) {
    sh.x_ready[threadIdx.x] = -1;
    sh.local_done[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    sh.err = 0;
    sh.next_item = 0;
  }
  __syncthreads();

  // This workgroup's share: in range mode (a list without dependencies) the
  // row-steps [ra, rb) of all GEMVs laid end to end, which lie in GEMVs j0..j1;
  // otherwise an even share of every GEMV (j0 = 0, j1 = n - 1).
  int ra = 0, rb = 0, j0 = 0, j1 = n - 1;
  if (ranges) {
    const int4 rr = ranges[wg];
    ra = __builtin_amdgcn_readfirstlane(rr.x);
    rb = __builtin_amdgcn_readfirstlane(rr.y);
    j0 = __builtin_amdgcn_readfirstlane(rr.z);
    j1 = __builtin_amdgcn_readfirstlane(rr.w);
  }
  // row-steps [lo, hi) of a GEMV in this workgroup: sbase is the GEMV's first
  // row-step in the concatenation when srem < 0 (range mode), else the even split
  auto item_range = [&](int sbase, int srem, int steps, int flags, int& lo, int& hi) {
    if (srem < 0) {
      lo = min(max(ra - sbase, 0), steps);
      hi = min(max(rb - sbase, 0), steps);
    } else if (flags & kPairs) {
      lo = min(2 * wg_step(sbase, srem, wg), steps);
      hi = min(2 * wg_step(sbase, srem, wg + 1), steps);
    } else {
      lo = wg_step(sbase, srem, wg);
      hi = wg_step(sbase, srem, wg + 1);
    }
  };

  if (wave < kSync) {
    // ----------------------------------------------------------- sync waves
    // Sync wave `wave` owns this workgroup's GEMVs k = j0 + wave (mod kSync): it
    // stages their x and copies out / publishes their y.  NX is a multiple of
    // kSync, so GEMV k and the GEMV k - NX whose buffer it reuses have the same
    // owner.  Buffers and counters are indexed from j0.
    const int me = wave;
    const Nibbles nbs = make_nibbles();
    int next_fin = j0 + me;            // next own GEMV to copy out and publish
    auto complete = [&](int i) {
      return (unsigned)lds_load(&sh.local_done[(i - j0) % NX]) >=
             (unsigned)kCompute * (unsigned)((i - j0) / NX + 1);
    };
    auto finish_one = [&](int i) {
      const StepDesc& d = D[i];
      const int b = (i - j0) % NX;
      const int rps = 64 >> d.lpr_log2;
      int lo, hi;
      item_range(d.sbase, d.srem, d.steps, d.flags, lo, hi);
      const int r0 = lo * rps;
      int r1 = hi * rps;
      if (r1 > d.N) r1 = d.N;
      const uint16_t* yb = ybuf + b * ybuf_rows;
      if (d.flags & kTagOut) {
        // the rows as tagged pairs for the GEMV that reads them: one 64-bit store
        // per pair (two values and the epoch land together), written through to
        // the coherence point; nothing waits for them here (r0 is even)
        const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<unsigned char*>(ctl) + d.tag_out, 0, 0x7FFFFFFF, kRsrcFlags);
        for (int q = (r0 >> 1) + lane; 2 * q < r1; q += 64) {
          const uint32_t lo16 = yb[2 * q - r0];
          const uint32_t hi16 = 2 * q + 1 < r1 ? yb[2 * q + 1 - r0] : 0u;
          const u32x2_g t = {lo16 | (hi16 << 16), epoch};
          __builtin_amdgcn_raw_buffer_store_b64(t, rt, 8 * q, 0, kCoherent);
        }
      }
      if (!(d.flags & kPublish)) {
        Q4_GLOBAL uint16_t* Y = gptr_mut(d.Y);
        for (int r = r0 + lane; r < r1; r += 64) Y[r] = yb[r - r0];
      } else {
        // device-coherent stores (written through to the coherence point), then
        // wait for them and count this workgroup in: no cache-wide write-back
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            d.Y, 0, 0x7FFFFFFF, kRsrcFlags);
        for (int r = r0 + lane; r < r1; r += 64)
          __builtin_amdgcn_raw_buffer_store_b16(yb[r - r0], ry, 2 * r, 0, kCoherent);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (lane == 0)
          __hip_atomic_fetch_add(&done[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    // finish own GEMVs <= last in order; block: wait for each to complete locally,
    // otherwise stop at the first one that has not
    auto finish_upto = [&](int last, bool block) {
      while (next_fin <= last && next_fin <= j1) {
        if (!complete(next_fin)) {
          if (!block) return;
          // a long sleep: polling issues vector instructions that the
          // compute waves on this SIMD would otherwise use
          for (unsigned it = 0; !complete(next_fin); ++it) {
            if (it > kSpinLimit / 8) { report_error(ctl, kErrLocal, next_fin); break; }
            __builtin_amdgcn_s_sleep(8);
          }
        }
        finish_one(next_fin);
        next_fin += kSync;
      }
    };
    for (int k = j0 + me; k <= j1; k += kSync) {
      const StepDesc& d = D[k];
      const int G = d.G, nblk = 4 * G;
      finish_upto(k - kSync, false);             // publish what is already complete
      if (k - j0 >= NX) finish_upto(k - NX, true);   // buffer (k - j0) % NX is free again
      const bool tagged = (d.flags & kTagIn) != 0;
      const bool coherent = d.dep >= 0 && !tagged;
      if (tagged) {
        // this workgroup's own share of the producer comes first (the others
        // finish at about the same time): poll the pairs only after it
        for (unsigned it = 0; d.dep >= j0 && !complete(d.dep); ++it) {
          if (it > kSpinLimit) { report_error(ctl, kErrTag, k); break; }
          finish_upto(k - kSync, false);
          __builtin_amdgcn_s_sleep(1);
        }
        // every own GEMV up to the producer is complete here: publish them before
        // polling (other workgroups' shares of the producer may depend on them)
        finish_upto(k - kSync, false);
      }
      if (coherent) {
        if ((d.dep - j0) % kSync == me) finish_upto(d.dep, true);
        for (unsigned it = 0;
             __hip_atomic_load(&done[d.dep], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             (unsigned)nwg;
             ++it) {
          if (it > kSpinLimit) { report_error(ctl, kErrCounter, k); break; }
          finish_upto(k - kSync, false);         // others may be waiting for those
          __builtin_amdgcn_s_sleep(1);
        }
      }
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(d.X), 0, 0x7FFFFFFF, kRsrcFlags);
      const Q4_GLOBAL u32x4_g* X = (const Q4_GLOBAL u32x4_g*)d.X;
      const int b = (k - j0) % NX;
      uint4* xb = xbuf + b * 4 * maxG;
      float* cb = cbuf + b * maxG;
      // x_k in (at most) two batches of 8 blocks per lane: one round trip for
      // K <= 4096.  With the feed-forward glue, x is [gate | up] (block i of h
      // from blocks i and nblk + i) in batches of 4 blocks per lane.
      const bool silu = (d.flags & kSiluMul) != 0;
      const int batch = silu ? 4 * 64 : 8 * 64;
      for (int i0 = 0; i0 < nblk; i0 += batch) {
        uint4 v[8];
        if (silu) {
          // h = fp16(silu(gate) * up), formed as soon as both blocks are in
          auto glue = [&](uint4 g4, uint4 u4) {
            const h8_t g = bits<h8_t>(g4), uu = bits<h8_t>(u4);
            h8_t h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = silu_mul_h(g[e], uu[e]);
            return bits<uint4>(h);
          };
          if (tagged) {
            const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<unsigned char*>(ctl) + d.tag_in, 0, 0x7FFFFFFF, kRsrcFlags);
            unsigned pend = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (i0 + u * 64 + lane < nblk) pend |= 1u << u;
            for (unsigned it = 0;; ++it) {
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (pend & (1u << u)) {
                  const int i = i0 + u * 64 + lane, iu = i + nblk;
                  const u32x4_g a = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * i, 0, kCoherent);
                  const u32x4_g c2 = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * i + 16, 0, kCoherent);
                  const u32x4_g e = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * iu, 0, kCoherent);
                  const u32x4_g f = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * iu + 16, 0, kCoherent);
                  if (a[1] == epoch && a[3] == epoch && c2[1] == epoch && c2[3] == epoch &&
                      e[1] == epoch && e[3] == epoch && f[1] == epoch && f[3] == epoch) {
                    v[u] = glue(make_uint4(a[0], a[2], c2[0], c2[2]),
                                make_uint4(e[0], e[2], f[0], f[2]));
                    pend &= ~(1u << u);
                  }
                }
              }
              if (!__builtin_amdgcn_ballot_w64(pend != 0u)) break;
              if (it > kTagSpinLimit) { report_error(ctl, kErrTag, k); break; }
              finish_upto(k - kSync, false);
              __builtin_amdgcn_s_sleep(1);
            }
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int i = i0 + u * 64 + lane;
              if (i < nblk) {
                u32x4_g a, e;
                if (coherent) {
                  a = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * i, 0, kCoherent);
                  e = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * (i + nblk), 0, kCoherent);
                } else {
                  a = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * i, 0, 0);
                  e = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * (i + nblk), 0, 0);
                }
                v[u] = glue(make_uint4(a[0], a[1], a[2], a[3]), make_uint4(e[0], e[1], e[2], e[3]));
              }
            }
          }
        } else if (tagged) {
          // block i = tagged pairs 4i .. 4i + 3 (two 16-byte loads from the
          // coherence point); a block is taken once all four carry this call's
          // epoch, and re-read until then
          const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
              reinterpret_cast<unsigned char*>(ctl) + d.tag_in, 0, 0x7FFFFFFF, kRsrcFlags);
          unsigned pend = 0;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (i0 + u * 64 + lane < nblk) pend |= 1u << u;
          for (unsigned it = 0;; ++it) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (pend & (1u << u)) {
                const int i = i0 + u * 64 + lane;
                const u32x4_g a = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * i, 0, kCoherent);
                const u32x4_g c2 = __builtin_amdgcn_raw_buffer_load_b128(rt, 32 * i + 16, 0, kCoherent);
                if (a[1] == epoch && a[3] == epoch && c2[1] == epoch && c2[3] == epoch) {
                  v[u] = make_uint4(a[0], a[2], c2[0], c2[2]);
                  pend &= ~(1u << u);
                }
              }
            }
            if (!__builtin_amdgcn_ballot_w64(pend != 0u)) break;
            if (it > kTagSpinLimit) { report_error(ctl, kErrTag, k); break; }
            finish_upto(k - kSync, false);
            __builtin_amdgcn_s_sleep(1);
          }
        } else if (coherent) {
          // x may have been written by other workgroups in this launch: read it
          // from the coherence point, past every cache
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 64 + lane;
            if (i < nblk) {
              const u32x4_g t = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * i, 0, kCoherent);
              v[u] = make_uint4(t[0], t[1], t[2], t[3]);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 64 + lane;
            if (i < nblk) {
              const u32x4_g t = X[i];
              v[u] = make_uint4(t[0], t[1], t[2], t[3]);
            }
          }
        }
        // pair-order the blocks into plane j = word j
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 64 + lane;
          if (u * 64 < batch && i < nblk) xb[(i & 3) * maxG + (i >> 2)] = pair_order(v[u]);
        }
      }
      // per group the offset term: the compute waves' chain over codes all 7
      // with this x (see nibble_group_dot), read back from the planes just written
      wait_lds();
      {
        const uint4 w7 = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
        const uint4 w1 = make_uint4(0x11111111u, 0x11111111u, 0x11111111u, 0x11111111u);
        const bool q3 = (d.flags & kQ3) != 0;
        const bool aff = AFF && (d.flags & kAffine) != 0;
        float* const sb = sbuf + b * maxG;
        for (int g = lane; g < G; g += 64) {
          uint4 xq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) xq[q] = xb[q * maxG + g];
          // q3f16_1: the same chain over codes all 3 (q3_group_dot)
          cb[g] = q3 ? q3_group_dot(kQ3Zero0, kQ3Zero1, kQ3Zero2, xq, kQ3MaskA, kQ3MaskB)
                     : nibble_group_dot(w7, xq, nbs);
          // affine: also the chain over codes all 1, 2^-20 times the group's sum of
          // x, for its (b + 7 s) term
          if (aff) sb[g] = nibble_group_dot(w1, xq, nbs);
        }
      }
      // groups past G up to the padded count read x = 0 and bias 0, so the
      // duplicated weights loaded for them contribute nothing
      const int Gp = (1 << d.lpr_log2) * d.C;
      for (int i = 4 * G + lane; i < 4 * Gp; i += 64) {
        xb[(i & 3) * maxG + (i >> 2)] = make_uint4(0u, 0u, 0u, 0u);
        if ((i & 3) == 0) {
          cb[i >> 2] = 0.f;
          if (AFF && (d.flags & kAffine)) sbuf[b * maxG + (i >> 2)] = 0.f;
        }
      }
      wait_lds();
      if (lane == 0) __hip_atomic_store(&sh.x_ready[b], k, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    finish_upto(j1, true);
    if (me == 0) {
      // every compute wave has signalled the last GEMV (so none will still set
      // the error word) once the owner of GEMV j1 is done; wave 0 waits for
      // the last completion before reading it
      for (unsigned it = 0; j0 <= j1 && !complete(j1); ++it) {
        if (it > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) {
        const int e = lds_load(&sh.err);
        if (e) report_error(ctl, kErrX, e - 1);
      }
    }
  } else {

  // -------------------------------------------------------------- compute waves
  const Nibbles nb = make_nibbles();
  // the q3f16_1 field masks in registers (q3_group_dot)
  uint32_t q3ma = kQ3MaskA, q3mb = kQ3MaskB;
  asm volatile("" : "+v"(q3ma), "+v"(q3mb));
  // Issue cursor.  A workgroup's items of all GEMVs, in list order, form one
  // sequence.  In range mode a wave takes the next B of them from an LDS counter
  // whenever it issues a burst, so waves that get their loads back sooner take
  // more items and all of them run out of work together (a fixed deal leaves
  // the last waves streaming alone while the others idle).  Either way a wave's
  // items come in sequence order and the cursor only moves forward.  It
  // keeps the current GEMV's descriptor in (scalar) registers: the table is read
  // only at GEMV transitions, never per item.
  struct Cursor {
    const Q4_GLOBAL uint4* W;
    const Q4_GLOBAL uint16_t* S;
    int j, s0, cnt, first;       // GEMV, its first row-step here, its item count, and
                                 // the sequence index of its first item
    int N, G, lg, C, r0;         // its shape, and its first row in this workgroup
    int q3;                      // q3f16_1 words (12 bytes per group)
    int aff;                     // affine: 0 none, 1 bf16 scales and biases, 2 fp16
    const Q4_GLOBAL uint16_t* Bs;   // affine: the biases
    int vo[4];                   // this lane's byte offset of each slot in an item's words
                                 // (16 bytes per group; q3f16_1 loads take 3/4 of it)
  } cu;
#pragma unroll
  for (int t = 0; t < 4; ++t) cu.vo[t] = 0;
  auto load = [&](int j) {       // make GEMV j the cursor's
    const CursorDesc d = read_desc(D + j);
    int s0, s1;
    item_range(d.sbase, d.srem, d.steps, d.flags, s0, s1);
    cu.W = d.W;
    cu.S = d.S;
    cu.N = d.N;
    cu.G = d.G;
    cu.lg = d.lg;
    cu.C = d.C;
    cu.q3 = (d.flags & kQ3) != 0;
    cu.aff = !AFF || !(d.flags & kAffine) ? 0 : (d.flags & kAffineF16) ? 2 : 1;
    cu.Bs = cu.aff ? read_bias(D + j) : nullptr;
    cu.j = j;
    cu.s0 = s0;
    cu.cnt = s1 - s0;
    cu.r0 = s0 * (64 >> d.lg);
    const int li = lane & ((1 << d.lg) - 1), g0 = (lane >> d.lg) * d.G + li;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool in = t < d.C && li + (t << d.lg) < d.G;
      // a slot past the row's groups (padded rows, or t >= C) takes an offset
      // of 2 GiB - 16: past the end of the resource (which is capped at 4 GiB -
      // 16) unless more than 2 GiB of the matrix follow the item, and then still
      // inside it; it is masked off or never consumed.  Reading zeros instead of
      // re-reading a real group keeps the slot off the memory system.
      cu.vo[t] = in ? (g0 + (t << d.lg)) * 16 : 0x7FFFFFF0;
    }
  };
  cu.j = j0;
  cu.first = 0;
  cu.cnt = 0;
  if (j0 <= j1) load(j0);
  // move the cursor to the GEMV holding sequence item `it` (past j1: none)
  auto seek = [&](int it) {
    while (cu.j <= j1 && it >= cu.first + cu.cnt) {
      cu.first += cu.cnt;
      if (++cu.j <= j1) load(cu.j);
    }
  };
  // The first of the next B sequence items of this wave, which are `stride`
  // apart.  Range mode: the next B items of the sequence, from the LDS counter
  // (the value is lane 0's: read it with readfirstlane where it is used, so the
  // LDS round trip overlaps other work).  Spread mode: a fixed round-robin deal
  // (wave c takes items c, c + 12, ...).  There a workgroup's share of a GEMV is
  // a few items that often wait for the GEMV's input, and the deal spreads them
  // over as many waves as possible, where claiming in twos would let one wave
  // take two of them in a row -- in a chain of dependent GEMVs every GEMV waits
  // for its slowest wave.
  const bool claim = ranges != nullptr;
  const int stride = claim ? 1 : kCompute;
  int dealt = wave - kSync;
  auto take = [&]() {
    int v = dealt;
    if (claim) {
      if (lane == 0)
        v = __hip_atomic_fetch_add(&sh.next_item, B, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      dealt += B * kCompute;
    }
    return v;
  };

  auto wait_x = [&](int j) {
    for (unsigned it = 0; lds_load(&sh.x_ready[(j - j0) % NX]) != j; ++it) {
      if (it > kSpinLimit) {
        __hip_atomic_store(&sh.err, j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };
  int cur = j0;                   // GEMVs [j0, cur) have been signalled by this wave
  auto signal_upto = [&](int j) { // signal completion of GEMVs [cur, j)
    for (; cur < j; ++cur) {
      wait_x(cur);
      wait_lds();                 // this wave's y rows of `cur` are in LDS
      if (lane == 0) __hip_atomic_fetch_add(&sh.local_done[(cur - j0) % NX], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  };

  // Bursts of B items: all loads of a burst are issued before any is consumed,
  // so no loaded value crosses the loop's back edge (the compiler then waits
  // exactly for the item being consumed).  Every issue is exactly eight loads
  // (four dwordx4 + four ushort).  They are buffer loads: the item's first row is
  // the base of a buffer resource (scalar arithmetic) bounded by the end of the
  // matrix, so rows past it read as zero without touching memory; a lane's offset
  // within an item is fixed per GEMV and a slot's offset is a scalar, so issuing
  // costs no vector arithmetic.  Slots past a lane's groups point past the
  // buffer (no memory access); items past the end of the list use an empty
  // resource.
  const Q4_GLOBAL uint4* const W_last = read_desc(D + (n - 1)).W;
  // One burst of B items: the loads of every item (as loaded registers) and what
  // consuming them needs.
  struct Burst {
    uint4 rw[B][4];
    uint16_t rs[B][4];           // scales; affine: the pair's scale (even lane) or bias (odd)
    int rj[B], rrow[B], rN[B], rG[B], rlg[B], rC[B], rr0[B], rq[B], ra[B];
  };
  auto issue = [&](Burst& U, int it0) {   // items it0 + p * stride
#pragma unroll
    for (int p = 0; p < B; ++p) {
      seek(it0 + p * stride);
      const bool live = cu.j <= j1;
      const int lg = live ? cu.lg : 2;
      const int G = live ? cu.G : 1;
      const int C = live ? cu.C : 1;
      const int row0 = live ? (cu.s0 + it0 + p * stride - cu.first) * (64 >> lg) : 0;
      const bool q3 = live && cu.q3;
      const int aff = live ? cu.aff : 0;
      const uint64_t left = live ? (uint64_t)(cu.N - row0) * (uint64_t)G : 0;   // groups
      const uint64_t gb = q3 ? 12 : 16;                                         // bytes per group
      const uint32_t nw = left * gb < 0xFFFFFFF0ull ? (uint32_t)(left * gb) : 0xFFFFFFF0u;
      // scales: 2 bytes per group, or (affine) per two groups
      const uint64_t sb = aff ? left : left * 2;
      const uint32_t ns = sb < 0xFFFFFFF0ull ? (uint32_t)sb : 0xFFFFFFF0u;
      const Q4_GLOBAL uint8_t* wrow =
          (const Q4_GLOBAL uint8_t*)cu.W + (int64_t)row0 * G * (int64_t)gb;
      const __amdgpu_buffer_rsrc_t bw = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(live ? (const uint8_t*)wrow : (const uint8_t*)W_last),
          0, (int)nw, kRsrcFlags);
      const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(live ? (const uint16_t*)(cu.S + (int64_t)row0 * (aff ? G / 2 : G))
                                     : (const uint16_t*)W_last),
          0, (int)ns, kRsrcFlags);
      // AFF: the scales (and biases) through per-lane addresses instead; a lane
      // with nothing to read (a slot past the row, a row past the matrix, an item
      // past the end) reads 2 bytes at W_last, which nothing consumes
      const bool row_in = live && row0 + (lane >> lg) < cu.N;
      const Q4_GLOBAL uint16_t* srow = cu.S + (int64_t)row0 * (aff ? G / 2 : G);
      const Q4_GLOBAL uint16_t* brow = aff ? cu.Bs + (int64_t)row0 * (G / 2) : srow;
      // Per-lane slot offsets are fixed per GEMV (the cursor's).  Only this
      // per-lane part of a buffer address is range-checked, so the scalar offset
      // stays 0; lanes past the end of the matrix (or of an empty resource) read
      // zeros without a memory access.
      // (q3f16_1: one 12-byte load per group at 3/4 of the slot's 16-byte offset;
      // the 2 GiB - 16 of a slot past the row becomes 1.5 GiB - 12, past the
      // resource unless more than 1.5 GiB of the matrix follow the item)
      if (q3) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int wo = (cu.vo[t] >> 1) + (cu.vo[t] >> 2);
          const u32x3_g v = __builtin_amdgcn_raw_buffer_load_b96(bw, wo, 0, kNonTemporal);
          U.rw[p][t] = make_uint4(v[0], v[1], v[2], 0u);
          U.rs[p][t] = __builtin_amdgcn_raw_buffer_load_b16(bs, cu.vo[t] >> 3, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4_g v = __builtin_amdgcn_raw_buffer_load_b128(bw, cu.vo[t], 0, kNonTemporal);
          U.rw[p][t] = make_uint4(v[0], v[1], v[2], v[3]);
          if (AFF) {
            // one 2-byte load per slot: the group's scale, or (affine) the lane of
            // the pair's even group takes the pair's scale and the lane of its odd
            // group (the next lane of the same row) the pair's bias; the two swap
            // them when the burst is consumed.  Slot offset / 16 is the group.
            const bool in = row_in && cu.vo[t] != 0x7FFFFFF0;
            const int el = aff ? cu.vo[t] >> 5 : cu.vo[t] >> 4;
            const Q4_GLOBAL uint16_t* a =
                in ? (aff && (lane & 1) ? brow : srow) + el : (const Q4_GLOBAL uint16_t*)W_last;
            U.rs[p][t] = *a;
          } else {
            U.rs[p][t] = __builtin_amdgcn_raw_buffer_load_b16(bs, cu.vo[t] >> 3, 0, 0);
          }
        }
      }
      U.rj[p] = live ? cu.j : -1;
      U.rrow[p] = row0;
      U.rN[p] = cu.N;
      U.rG[p] = G;
      U.rlg[p] = lg;
      U.rC[p] = C;
      U.rr0[p] = cu.r0;
      U.rq[p] = q3;
      U.ra[p] = aff;
    }
  };
  // Consume a burst in item order; false once an item past the end is reached.
  auto consume = [&](Burst& U) -> bool {
    // All items of the burst in one GEMV (the common case): x of each group is
    // read from LDS once and used for all B rows, which also gives B independent
    // dot-product chains.
    if (U.rj[B - 1] >= 0 && U.rj[0] == U.rj[B - 1]) {
      const int j = U.rj[0];
      signal_upto(j);
      wait_x(j);
      const int lg = U.rlg[0], lpr = 1 << lg;
      const int li = lane & (lpr - 1);
      const int xi = (j - j0) % NX;
      const uint4* xb = xbuf + xi * 4 * maxG + li;
      const float* cb = cbuf + xi * maxG + li;
      if (U.rC[0] * lpr > U.rG[0]) {      // padded rows: slots past G hold other data
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool ok = li + lpr * t < U.rG[0];
#pragma unroll
          for (int p = 0; p < B; ++p) {
            U.rs[p][t] = ok ? U.rs[p][t] : (uint16_t)0;
          }
        }
      }
      float acc[B];
#pragma unroll
      for (int p = 0; p < B; ++p) acc[p] = 0.f;
      if (AFF && U.ra[0]) {
        // affine, per group: s * sum((q - 7) x) + (b + 7 s) * sum(x), the first as
        // the q4f16_1 groups form it (so centred groups cancel before the scaling),
        // both in the chain's 2^-20 units; 7 s is exact in fp32
        const bool f16 = U.ra[0] == 2;
        const float* sb = sbuf + xi * maxG + li;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < U.rC[0]) {
            uint4 x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * t];
            const float off = cb[lpr * t], sx = sb[lpr * t];
#pragma unroll
            for (int p = 0; p < B; ++p) {
              const float pd = nibble_group_dot(U.rw[p][t], x, nb) - off;
              float sc, bi;
              pair_values(U.rs[p][t], f16, sc, bi);
              acc[p] = __builtin_fmaf(pd, sc, acc[p]);
              acc[p] = __builtin_fmaf(sx, __builtin_fmaf(7.f, sc, bi), acc[p]);
            }
          }
        }
      } else
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < U.rC[0]) {
          uint4 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * t];
          const float off = cb[lpr * t];
#pragma unroll
          for (int p = 0; p < B; ++p) {
            const uint4 w = U.rw[p][t];
            const float pd =
                (U.rq[0] ? q3_group_dot(w.x, w.y, w.z, x, q3ma, q3mb) : nibble_group_dot(w, x, nb)) -
                off;
            acc[p] = __builtin_fmaf(pd, (float)bits<_Float16>(U.rs[p][t]), acc[p]);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < B; ++p) {
        // q3_group_dot is in the products' own units
        const float r = team_sum_lg(acc[p], lg) * (U.rq[0] ? 1.f : kDotUnit);
        const int row = U.rrow[p] + (lane >> lg);
        if (li == 0 && row < U.rN[p])
          ybuf[xi * ybuf_rows + (row - U.rr0[p])] = bits<uint16_t>((_Float16)r);
      }
      return true;
    }
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const int j = U.rj[p];
      if (j < 0) return false;
      signal_upto(j);
      wait_x(j);
      const int lg = U.rlg[p], lpr = 1 << lg;
      const int li = lane & (lpr - 1);
      const int row = U.rrow[p] + (lane >> lg);
      const int xi = (j - j0) % NX;
      const uint4* xb = xbuf + xi * 4 * maxG + li;
      const float* cb = cbuf + xi * maxG + li;
      if (U.rC[p] * lpr > U.rG[p]) {      // padded rows: slots past G hold other data
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          U.rs[p][t] = li + lpr * t < U.rG[p] ? U.rs[p][t] : (uint16_t)0;
        }
      }
      float acc = 0.f;
      if (AFF && U.ra[p]) {
        const bool f16 = U.ra[p] == 2;
        const float* sb = sbuf + xi * maxG + li;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < U.rC[p]) {
            uint4 x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * t];
            const float pd = nibble_group_dot(U.rw[p][t], x, nb) - cb[lpr * t];
            float sc, bi;
            pair_values(U.rs[p][t], f16, sc, bi);
            acc = __builtin_fmaf(pd, sc, acc);
            acc = __builtin_fmaf(sb[lpr * t], __builtin_fmaf(7.f, sc, bi), acc);
          }
        }
      } else
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < U.rC[p]) {
          uint4 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * t];
          const uint4 w = U.rw[p][t];
          const float pd =
              (U.rq[p] ? q3_group_dot(w.x, w.y, w.z, x, q3ma, q3mb) : nibble_group_dot(w, x, nb)) -
              cb[lpr * t];
          acc = __builtin_fmaf(pd, (float)bits<_Float16>(U.rs[p][t]), acc);
        }
      }
      acc = team_sum_lg(acc, lg) * (U.rq[p] ? 1.f : kDotUnit);
      if (li == 0 && row < U.rN[p])
        ybuf[xi * ybuf_rows + (row - U.rr0[p])] = bits<uint16_t>((_Float16)acc);
    }
      return true;
  };
  // All loads of a burst are issued before any is consumed, so no loaded value
  // crosses the loop's back edge and every issue is the same eight loads per
  // item: the compiler then waits exactly for the item being consumed.
  int next = take();
  while (true) {
    Burst U;
    issue(U, __builtin_amdgcn_readfirstlane(next));
    next = take();
    if (!consume(U)) break;
  }
    signal_upto(j1 + 1);
  }

  // Leave the counters zeroed for the next call and hand it the epoch: the last
  // workgroup to get here (every other one has finished with them, and every
  // one read the epoch when it started) does it.
  __syncthreads();
  if (wave == 0) {
    unsigned old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(ctl + kCtlExit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == (unsigned)nwg - 1u) {
      for (int i = lane; i < n; i += 64)
        __hip_atomic_store(done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) {
        __hip_atomic_store(ctl + kCtlExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctl + kCtlEpoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__global__ void k_zero(unsigned* __restrict__ p, size_t count) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// A piece of a table passed by value in the kernel arguments.
constexpr int kPieceWords = 240;
struct TablePiece {
  uint32_t w[kPieceWords];
};
__global__ void k_put(uint32_t* __restrict__ dst, TablePiece piece, int count) {
  if ((int)threadIdx.x < count) dst[threadIdx.x] = piece.w[threadIdx.x];
}

constexpr int kBurst = 2;

}  // namespace

hipError_t write_table(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes % 4) return hipErrorInvalidValue;
  const uint32_t* w = static_cast<const uint32_t*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  const size_t words = bytes / 4;
  for (size_t i = 0; i < words; i += kPieceWords) {
    const int c = (int)std::min<size_t>(kPieceWords, words - i);
    TablePiece piece;
    std::memcpy(piece.w, w + i, (size_t)c * 4);
    hipLaunchKernelGGL(k_put, dim3(1), dim3(256), 0, s, d + i, piece, c);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t zero_words(void* dst, size_t words, hipStream_t s) {
  if (!words) return hipSuccess;
  const int blocks = (int)std::max<size_t>(1, std::min<size_t>(1024, words / 4096));
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, s, static_cast<unsigned*>(dst), words);
  return hipGetLastError();
}

StepPlan plan_step(const DeviceInfo& d, const StepLayer* layers, int64_t n, bool ordered,
                   bool tags) {
  StepPlan p;
  p.ok = false;
  if (n < 1) return p;
  p.grid = d.cus;
  p.desc.resize((size_t)n);
  int maxG = 1, ybuf_rows = 1;
  for (int64_t k = 0; k < n; ++k) {
    const StepLayer& L = layers[k];
    const int64_t G = L.K / 32;
    if (G > 256) return p;                    // rows beyond 4 groups per lane
    int lg = 2;
    while ((4 << lg) < G && lg < 6) ++lg;     // 2^lg lanes x 4 groups >= G
    const int lpr = 1 << lg;
    const int C = (int)((G + lpr - 1) / lpr);
    const int rps = 64 / lpr;
    StepDesc& s = p.desc[(size_t)k];
    s.W = reinterpret_cast<const uint4*>(L.words);
    s.S = L.scales;
    s.X = reinterpret_cast<const uint4*>(L.x);
    s.Y = L.y;
    s.N = (int)L.N;
    s.G = (int)G;
    s.lpr_log2 = lg;
    s.C = C;
    s.steps = (int)((L.N + rps - 1) / rps);
    s.dep = -1;
    const bool aff = L.format == Q4_FMT_AF4_G64 || L.format == Q4_FMT_AF4_G64_F16;
    s.flags = (L.x_op ? kSiluMul : 0) | (L.format == Q4_FMT_Q3F16_1 ? kQ3 : 0) |
              (aff ? kAffine : 0) | (L.format == Q4_FMT_AF4_G64_F16 ? kAffineF16 : 0);
    s.tag_in = s.tag_out = 0;
    s.Bs = aff ? L.biases : nullptr;
    if (aff) p.affine = true;
    s.sbase = s.steps / p.grid;
    s.srem = s.steps % p.grid;
    if (lpr * C > maxG) maxG = lpr * C;         // padded group count
    const int rows_wg = ((s.steps + p.grid - 1) / p.grid) * rps;
    if (rows_wg > ybuf_rows) ybuf_rows = rows_wg;
  }
  // Dependencies.  Descriptor k conflicts with an earlier h whose y overlaps k's x
  // (k reads what h writes) or k's y (both write it), and with an earlier g whose x
  // overlaps k's y (k overwrites what g reads); ordered, also with k - 1.
  //  * Hand-over: when k's only conflict is one h whose y holds all of k's x (at
  //    an even element offset), h also writes its y as epoch-tagged pairs to the
  //    workspace and k reads x from those as soon as they are there: no
  //    completion counter, no wait for the rest of h.
  //  * Otherwise k waits for the completion counter of its latest conflict.  A
  //    workgroup publishes a GEMV only after staging the x of every GEMV before
  //    it, and stages x only after its own counter wait, so that wait also covers
  //    a writer reached from it through counter waits (and every reader before
  //    it); a list with a writer not covered so runs one kernel per GEMV.
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
  };
  std::vector<int> tag_src((size_t)n, -1);
  for (int64_t k = 1; k < n; ++k) {
    const StepLayer& Lk = layers[k];
    int last = ordered ? (int)k - 1 : -1, raw_h = -1, raw_n = 0;
    bool other = false;
    std::vector<int> writers;
    for (int64_t i = k - 1; i >= 0; --i) {
      const StepLayer& Li = layers[i];
      const bool raw = overlap(Li.y, 2 * Li.N, Lk.x, 2 * Lk.x_cols());
      const bool waw = overlap(Li.y, 2 * Li.N, Lk.y, 2 * Lk.N);
      const bool war = overlap(Li.x, 2 * Li.x_cols(), Lk.y, 2 * Lk.N);
      if (raw || waw) writers.push_back((int)i);
      if (raw) { ++raw_n; raw_h = (int)i; }
      if (waw || war) other = true;
      if ((raw || waw || war) && (int)i > last) last = (int)i;
    }
    StepDesc& sk = p.desc[(size_t)k];
    if (tags && raw_n == 1 && !other && (!ordered || raw_h == (int)k - 1)) {
      const uintptr_t y0 = reinterpret_cast<uintptr_t>(layers[raw_h].y);
      const uintptr_t x0 = reinterpret_cast<uintptr_t>(Lk.x);
      if (x0 >= y0 && x0 + 2 * (uintptr_t)Lk.x_cols() <= y0 + 2 * (uintptr_t)layers[raw_h].N &&
          (x0 - y0) % 4 == 0) {
        tag_src[(size_t)k] = raw_h;
        sk.dep = raw_h;
        sk.flags |= kTagIn;
        p.desc[(size_t)raw_h].flags |= kTagOut;
        p.cross_wg = true;
        continue;
      }
    }
    if (last < 0) continue;
    sk.dep = last;
    p.desc[(size_t)last].flags |= kPublish;
    p.cross_wg = true;
    for (int h : writers) {
      int i = last;
      while (i > h && !(p.desc[(size_t)i].flags & kTagIn) && p.desc[(size_t)i].dep >= 0)
        i = p.desc[(size_t)i].dep;
      if (i != h) return p;                     // not covered: one kernel per GEMV
    }
  }
  // tagged pairs: after the control block and the counters, one 256-byte aligned
  // run per producer; a producer with one row per row-step splits its rows over
  // the workgroups in pairs, so every workgroup's first row is even
  p.tag_base = (((size_t)kCtlWords + (size_t)n) * sizeof(unsigned) + 255) & ~(size_t)255;
  std::vector<size_t> tag_off((size_t)n, 0);
  size_t tag_end = p.tag_base;
  for (int64_t k = 0; k < n; ++k) {
    StepDesc& sk = p.desc[(size_t)k];
    if (!(sk.flags & kTagOut)) continue;
    tag_off[(size_t)k] = tag_end;
    tag_end += ((size_t)((sk.N + 1) / 2) * 8 + 255) & ~(size_t)255;
    if (sk.lpr_log2 == 6) {
      const int pairs = (sk.steps + 1) / 2;
      sk.flags |= kPairs;
      sk.sbase = pairs / p.grid;
      sk.srem = pairs % p.grid;
      const int rows_wg = 2 * ((pairs + p.grid - 1) / p.grid);
      if (rows_wg > ybuf_rows) ybuf_rows = rows_wg;
    }
  }
  if (tag_end > (size_t)INT32_MAX) return p;
  p.tag_bytes = tag_end - p.tag_base;
  for (int64_t k = 0; k < n; ++k) {
    StepDesc& sk = p.desc[(size_t)k];
    if (sk.flags & kTagOut) sk.tag_out = (int)tag_off[(size_t)k];
    if (sk.flags & kTagIn) {
      const int h = tag_src[(size_t)k];
      const uintptr_t off = reinterpret_cast<uintptr_t>(layers[k].x) -
                            reinterpret_cast<uintptr_t>(layers[h].y);
      sk.tag_in = (int)(tag_off[(size_t)h] + 2 * off);   // 8 bytes per 4 bytes of x
    }
  }
  p.maxG = maxG;
  const size_t lds_cap = d.lds_per_block - sizeof(int) * 32;
  auto lds_for = [&](int nx, int rows) {
    return (size_t)nx * ((size_t)4 * maxG * 16 + (size_t)maxG * 4 + (size_t)rows * 2 +
                         (p.affine ? (size_t)maxG * 4 : 0));
  };
  // Range mode: without dependencies, each workgroup streams one contiguous
  // stretch of the row-steps of all GEMVs laid end to end (balanced by weight
  // bytes), so it meets only a few GEMV boundaries instead of every one.
  if (!p.cross_wg) {
    std::vector<int64_t> first((size_t)n + 1), cum((size_t)n + 1);   // row-steps, bytes
    for (int64_t k = 0; k < n; ++k) {
      const StepDesc& s = p.desc[(size_t)k];
      const int64_t step_bytes = (int64_t)(64 >> s.lpr_log2) * s.G * ((s.flags & kQ3) ? 14 : 18);
      first[(size_t)k + 1] = first[(size_t)k] + s.steps;
      cum[(size_t)k + 1] = cum[(size_t)k] + step_bytes * s.steps;
    }
    const int64_t total = cum[(size_t)n];
    std::vector<int64_t> cut((size_t)p.grid + 1);
    for (int w = 0; w <= p.grid; ++w) {
      const int64_t target = (int64_t)(((__int128)total * w) / p.grid);
      int64_t k = std::upper_bound(cum.begin(), cum.end(), target) - cum.begin() - 1;
      if (k >= n) k = n - 1;
      const StepDesc& s = p.desc[(size_t)k];
      const int64_t step_bytes = (int64_t)(64 >> s.lpr_log2) * s.G * ((s.flags & kQ3) ? 14 : 18);
      int64_t st = (target - cum[(size_t)k]) / step_bytes;
      if (st > s.steps) st = s.steps;
      cut[(size_t)w] = w == p.grid ? first[(size_t)n] : first[(size_t)k] + st;
    }
    auto gemv_of = [&](int64_t item) {   // GEMV holding row-step `item`
      return (int)(std::upper_bound(first.begin(), first.end(), item) - first.begin() - 1);
    };
    std::vector<int> ranges((size_t)p.grid * 4);
    int rows = 8;
    bool fits = first[(size_t)n] < INT32_MAX;
    for (int w = 0; w < p.grid && fits; ++w) {
      const int64_t a = cut[(size_t)w], b = cut[(size_t)w + 1];
      int j0 = 1, j1 = 0;                  // empty
      if (b > a) {
        j0 = gemv_of(a);
        j1 = gemv_of(b - 1);
        for (int j = j0; j <= j1; ++j) {
          const StepDesc& s = p.desc[(size_t)j];
          const int64_t lo = std::max<int64_t>(a - first[(size_t)j], 0);
          const int64_t hi = std::min<int64_t>(b - first[(size_t)j], s.steps);
          rows = std::max<int64_t>(rows, (hi - lo) * (64 >> s.lpr_log2));
        }
      }
      ranges[(size_t)w * 4 + 0] = (int)a;
      ranges[(size_t)w * 4 + 1] = (int)b;
      ranges[(size_t)w * 4 + 2] = j0;
      ranges[(size_t)w * 4 + 3] = j1;
    }
    rows = (rows + 7) & ~7;
    if (fits && lds_for(4, rows) <= lds_cap) {
      p.nx = 4;
      p.ybuf_rows = rows;
      p.ranges = std::move(ranges);
      for (int64_t k = 0; k < n; ++k) {
        p.desc[(size_t)k].sbase = (int)first[(size_t)k];
        p.desc[(size_t)k].srem = -1;
      }
      p.lds_bytes = lds_for(4, rows);
      p.ok = true;
      return p;
    }
  }
  p.nx = kXBufs;
  p.ybuf_rows = (ybuf_rows + 7) & ~7;
  p.lds_bytes = lds_for(kXBufs, p.ybuf_rows);
  p.ok = p.lds_bytes <= lds_cap;
  return p;
}

StepLaunch step_launch_of(const StepPlan& p) {
  StepLaunch L{};
  L.kind = 1;
  L.n = (int)p.desc.size();
  L.grid = p.grid;
  L.M = 1;
  L.nx = p.nx;
  L.maxG = p.maxG;
  L.ybuf_rows = p.ybuf_rows;
  L.stage_off = -1;
  L.cross_wg = p.cross_wg;
  L.has_ranges = !p.ranges.empty();
  L.lds_bytes = (uint32_t)p.lds_bytes;
  L.affine = p.affine ? 1u : 0u;
  L.clear_bytes = p.tag_base + p.tag_bytes;
  L.table_off = (L.clear_bytes + 255) & ~(uint64_t)255;
  L.ranges_off = L.table_off + p.desc.size() * sizeof(StepDesc);
  L.table_bytes = p.desc.size() * sizeof(StepDesc) + p.ranges.size() * sizeof(int);
  L.ws_bytes = L.table_off + L.table_bytes;
  return L;
}

void step_table_bytes(const StepPlan& p, std::vector<uint8_t>* out) {
  const size_t db = p.desc.size() * sizeof(StepDesc);
  out->resize(db + p.ranges.size() * sizeof(int));
  std::memcpy(out->data(), p.desc.data(), db);
  if (!p.ranges.empty())
    std::memcpy(out->data() + db, p.ranges.data(), p.ranges.size() * sizeof(int));
}

namespace {
auto step_kernel(int nx, bool affine) {
  if (affine) return nx == 4 ? k_step<kBurst, 4, true> : k_step<kBurst, kXBufs, true>;
  return nx == 4 ? k_step<kBurst, 4, false> : k_step<kBurst, kXBufs, false>;
}
}  // namespace

hipError_t step_prepare(const StepLaunch& L) {
  if (L.lds_bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(step_kernel(L.nx, L.affine != 0)),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds_bytes);
}

hipError_t launch_step(const StepLaunch& L, void* ws, hipStream_t s) {
  unsigned* ctl = static_cast<unsigned*>(ws);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const StepDesc* desc = reinterpret_cast<const StepDesc*>(base + L.table_off);
  const int4* rg = L.has_ranges ? reinterpret_cast<const int4*>(base + L.ranges_off) : nullptr;
  auto kern = step_kernel(L.nx, L.affine != 0);
  int n = L.n, maxG = L.maxG, yr = L.ybuf_rows;
  // Only waits across workgroups need every workgroup resident at once; without
  // them (no descriptor depends on another) a plain launch does, and it costs
  // far less at the kernel boundary than a cooperative one.
  if (L.cross_wg) {
    void* args[] = {(void*)&desc, (void*)&n, (void*)&ctl, (void*)&maxG, (void*)&yr, (void*)&rg};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(L.grid),
                                      dim3(kStepThreads), args, L.lds_bytes, s);
  }
  hipLaunchKernelGGL(kern, dim3(L.grid), dim3(kStepThreads), L.lds_bytes, s, desc, n, ctl, maxG,
                     yr, rg);
  return hipGetLastError();
}

hipError_t step_occupancy(const StepPlan& p, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu,
      reinterpret_cast<const void*>(step_kernel(p.nx, p.affine)), kStepThreads, p.lds_bytes);
}

}  // namespace q4
