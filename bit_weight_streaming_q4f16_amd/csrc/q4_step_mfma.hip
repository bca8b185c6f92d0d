// Persistent decode-step kernel for small M (2..8 rows of X per GEMV): the whole
// layer list in one launch, each GEMV's weights read once for all M rows (the
// Splash page's batched decode: several tokens or sequences share one pass over
// the weights), the products on matrix cores.
//
// v_mfma_f32_16x16x32_f16 multiplies a 16 x 32 A by a 32 x 16 B.  Here A = the M
// rows of X over one 32-weight group (rows past M are zero) and B = the group of
// 16 weight rows, so one MFMA is one group of one 16-row tile and its per-group
// scale is applied exactly, in fp32, to the result.  The weights enter B as the
// exact fp16 values q - 7: one v_and_or_b32 per pair places two codes in fp16
// mantissas (1024 + q or 64 + q, as in the M = 1 kernels) and one packed fp16
// add of -1031 or -71 takes the offset off, exactly (q - 7 is in [-7, 8]); the
// MFMA's accumulator input is zero.  So a group whose codes are all 7 gives
// exactly zero, and integer codes times integer X give the exact integer.
//
// One workgroup of 16 waves per compute unit:
//  * 12 compute waves take this workgroup's 16-row tiles of every GEMV in list
//    order, dealt round-robin.  Where G is a multiple of 8 (and the scales
//    16-byte aligned) a tile streams in bursts of sixteen groups: the rows'
//    scales first, then four loads of 8 rows x 128 contiguous bytes, written
//    (eight groups at a time) to the wave's LDS stage as word planes and read
//    back as word c of eight groups of row r in lane (c, r), the B layout; the
//    next burst is issued as soon as the current one is in LDS.
//    Otherwise in bursts of kChunks chunks of four groups: per lane one dwordx4
//    (group c of row r, for lane = 16c + r) and one 8-byte load of the row's four
//    scales, and a 4 x 4 exchange between lanes r, r + 16, r + 32, r + 48 leaves
//    word c of each of the four groups in lane (c, r).  X comes from LDS;
//    results go to LDS.
//  * 4 sync waves, each owning every 4th GEMV: stage its X (pair-ordered) into
//    the GEMV's LDS region once the GEMVs it depends on are
//    complete on every workgroup and the region's previous user is finished,
//    copy finished rows of Y out, publish completion (as in the M = 1 kernel).
// LDS regions are planned on the host as a ring: a GEMV's region is reused only
// after the GEMVs that used it before are finished.
#include <algorithm>
#include <climits>
#include <cstring>

#include "q4_step_mfma.h"
#include "q4_device.h"

namespace q4 {
namespace {

constexpr int kWaves = kStepThreads / 64;   // 16
constexpr int kSync = 4;
constexpr int kCompute = kWaves - kSync;
constexpr int kSlots = 8;                   // x_ready slots: GEMVs up to 8 apart in flight
constexpr int kChunks = 4;                  // chunks (of four groups) per burst
constexpr int kStage = 2048;                // per compute wave: one staged burst (16 rows x 8 groups)
constexpr int kXRounds = 4;                 // (m, g) pairs of X per lane whose loads are in flight together
constexpr unsigned kSpinLimit = 1u << 24;
// Range mode: what a GEMV boundary inside a workgroup's stretch costs, in bytes of
// weights streamed.  Two neighbouring GEMVs' LDS regions (X, and y until copied
// out) rarely fit together at M = 8, so the second GEMV's X is staged only once the
// first is finished and copied out, and the compute waves wait; measured, that is
// about 19 us, what a compute unit's share of the bandwidth streams of 512 KB.
constexpr int64_t kBoundaryCost = 512 * 1024;
static_assert(kSlots % kSync == 0, "a GEMV and the one whose slot it reuses share an owner");


struct Shared {
  int x_ready[kSlots];    // GEMV whose X is staged, per slot (-1: none)
  int local_done[kSlots]; // compute-wave completions per slot (monotonic)
  int fin[kSync];         // highest GEMV each sync wave has finished (copied out)
  int err;
  int claim;              // range mode: tiles of the workgroup's stretch claimed so far
};

__device__ __forceinline__ int tile_of(int tbase, int trem, int wg) {
  return wg * tbase + (wg < trem ? wg : trem);
}

// The fields a compute wave needs, read with scalar loads (see the M = 1 kernel:
// ordinary loads of the table would become vector loads and drain the stream).
struct TileDesc {
  const Q4_GLOBAL uint4* W;
  const Q4_GLOBAL uint16_t* S;
  int N, G, tbase, trem, xoff;
};
__device__ __forceinline__ TileDesc read_desc(const MStepDesc* d) {
  u32x4_g ws;
  u32x8_s rest;        // N, G, tbase, trem, dep, signal, xoff, rel
  asm volatile(
      "s_load_dwordx4 %0, %2, 0x0\n\t"
      "s_load_dwordx8 %1, %2, 0x20\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(ws), "=&s"(rest)
      : "s"(d));
  static_assert(offsetof(MStepDesc, N) == 32 && offsetof(MStepDesc, tbase) == 40 &&
                    offsetof(MStepDesc, xoff) == 56,
                "descriptor offsets read by the compute waves");
  TileDesc r;
  r.W = (const Q4_GLOBAL uint4*)(((uint64_t)ws[1] << 32) | ws[0]);
  r.S = (const Q4_GLOBAL uint16_t*)(((uint64_t)ws[3] << 32) | ws[2]);
  r.N = (int)rest[0];
  r.G = (int)rest[1];
  r.tbase = (int)rest[2];
  r.trem = (int)rest[3];
  r.xoff = (int)rest[6];
  return r;
}

// LDS region of a GEMV (byte offsets from xoff): X planes [G][4][8] uint4 (rows m <
// M used; the fixed stride lets the reads of a burst use immediate offsets from one
// address), then y [M][rows] fp16 (rows: this workgroup's rows of the GEMV; the
// host sizes the region for the most any workgroup has).
__device__ __forceinline__ int ybuf_off(int, int G) { return 8 * G * 64; }

__global__ __launch_bounds__(kStepThreads) void k_step_mfma(const MStepDesc* __restrict__ D, int n,
                                                            int M, unsigned* __restrict__ ctl,
                                                            const int4* __restrict__ ranges,
                                                            int stage_off) {
  unsigned* const done = ctl + kCtlWords;       // completion counters
  extern __shared__ uint4 smem[];
  __shared__ Shared sh;
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x, nwg = gridDim.x;
  if (threadIdx.x < kSlots) {
    sh.x_ready[threadIdx.x] = -1;
    sh.local_done[threadIdx.x] = 0;
  }
  if (threadIdx.x < kSync) sh.fin[threadIdx.x] = -1;
  if (threadIdx.x == 0) {
    sh.err = 0;
    sh.claim = 0;
  }
  __syncthreads();

  // This workgroup's share (as in the M = 1 kernel): in range mode the tiles
  // [ra, rb) of all GEMVs laid end to end, lying in GEMVs j0..j1; otherwise an
  // even share of every GEMV.  Slots, owners and counters are indexed from j0.
  int ra = 0, rb = 0, j0 = 0, j1 = n - 1;
  if (ranges) {
    const int4 rr = ranges[wg];
    ra = __builtin_amdgcn_readfirstlane(rr.x);
    rb = __builtin_amdgcn_readfirstlane(rr.y);
    j0 = __builtin_amdgcn_readfirstlane(rr.z);
    j1 = __builtin_amdgcn_readfirstlane(rr.w);
  }
  // tiles [lo, hi) of a GEMV in this workgroup: tbase is the GEMV's first tile in
  // the concatenation when trem < 0 (range mode), else the even split
  auto tile_range = [&](int tbase, int trem, int N, int& lo, int& hi) {
    if (trem < 0) {
      const int tiles = (N + 15) / 16;
      lo = min(max(ra - tbase, 0), tiles);
      hi = min(max(rb - tbase, 0), tiles);
    } else {
      lo = tile_of(tbase, trem, wg);
      hi = tile_of(tbase, trem, wg + 1);
    }
  };

  auto complete = [&](int i) {        // every compute wave is past GEMV i here
    return (unsigned)lds_load(&sh.local_done[(i - j0) % kSlots]) >=
           (unsigned)kCompute * (unsigned)((i - j0) / kSlots + 1);
  };

  if (wave < kSync) {
    // ------------------------------------------------------------ sync waves
    const int me = wave;
    int next_fin = j0 + me;
    auto finish_one = [&](int i) {
      const MStepDesc& d = D[i];
      int t0, t1;
      tile_range(d.tbase, d.trem, d.N, t0, t1);
      const int r0 = t0 * 16;
      int r1 = t1 * 16;
      if (r1 > d.N) r1 = d.N;
      const int rows = (t1 - t0) * 16, nr = r1 - r0;
      const uint16_t* yb = reinterpret_cast<const uint16_t*>(lds + d.xoff + ybuf_off(M, d.G));
      if (nr > 0) {
        // Row by row of Y.  Where every row's run starts 16-byte aligned (Y 16-byte
        // aligned, N a multiple of 8; r0 is a multiple of 16, so nr is then a
        // multiple of 8 too) as 16-byte LDS reads and stores; otherwise one value
        // per lane and store.  (A workgroup's share of a large GEMV is thousands of
        // values per row of X, copied after its last tile: the step's tail.)
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(d.Y, 0, 0x7FFFFFFF, kRsrcFlags);
        const bool vec = (reinterpret_cast<uintptr_t>(d.Y) & 15u) == 0 && d.N % 8 == 0;
        for (int m = 0; m < M; ++m) {
          const uint16_t* src = yb + m * rows;
          const int dst = 2 * (m * d.N + r0);
          if (vec) {
            for (int v = lane; v < nr / 8; v += 64) {
              const uint4 t = *reinterpret_cast<const uint4*>(src + 8 * v);
              const u32x4_g tv = {t.x, t.y, t.z, t.w};
              if (d.signal)
                __builtin_amdgcn_raw_buffer_store_b128(tv, ry, dst + 16 * v, 0, kCoherent);
              else
                __builtin_amdgcn_raw_buffer_store_b128(tv, ry, dst + 16 * v, 0, 0);
            }
          } else {
            for (int r = lane; r < nr; r += 64) {
              if (d.signal)
                __builtin_amdgcn_raw_buffer_store_b16(src[r], ry, dst + 2 * r, 0, kCoherent);
              else
                __builtin_amdgcn_raw_buffer_store_b16(src[r], ry, dst + 2 * r, 0, 0);
            }
          }
        }
      }
      if (d.signal) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (lane == 0)
          __hip_atomic_fetch_add(&done[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_lds();
      if (lane == 0) lds_store(&sh.fin[me], i);
    };
    auto finish_upto = [&](int last, bool block) {
      while (next_fin <= last && next_fin <= j1) {
        if (!complete(next_fin)) {
          if (!block) return;
          for (unsigned it = 0; !complete(next_fin); ++it) {
            if (it > kSpinLimit / 8) { report_error(ctl, kErrLocal, next_fin); break; }
            __builtin_amdgcn_s_sleep(8);
          }
        }
        finish_one(next_fin);
        next_fin += kSync;
      }
    };
    // every GEMV <= i finished (copied out) by its owner; this workgroup has no
    // part in GEMVs before j0
    auto finished_upto = [&](int i) {
      for (int o = 0; o < kSync; ++o) {
        const int r = i - j0;
        const int last = r - ((r - o) % kSync + kSync) % kSync;   // largest <= r owned by o
        if (last >= 0 && lds_load(&sh.fin[o]) < j0 + last) return false;
      }
      return true;
    };
    for (int k = j0 + me; k <= j1; k += kSync) {
      const MStepDesc& d = D[k];
      const int G = d.G;
      finish_upto(k - kSync, false);
      if (k - j0 >= kSlots) finish_upto(k - kSlots, true);   // slot (k - j0) % kSlots is free
      if (d.rel >= 0) {
        for (unsigned it = 0; !finished_upto(d.rel); ++it) {
          if (it > kSpinLimit) { report_error(ctl, kErrRegion, k); break; }
          finish_upto(k - kSync, false);
          finish_upto(d.rel, false);
          __builtin_amdgcn_s_sleep(2);
        }
      }
      const bool coherent = d.dep >= 0;
      if (coherent) {
        if ((d.dep - j0) % kSync == me) finish_upto(d.dep, true);
        for (unsigned it = 0;
             __hip_atomic_load(&done[d.dep], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             (unsigned)nwg;
             ++it) {
          if (it > kSpinLimit) { report_error(ctl, kErrCounter, k); break; }
          finish_upto(k - kSync, false);
          __builtin_amdgcn_s_sleep(1);
        }
      }
      // X rows m < M: lane takes (m, g) pairs, kXRounds of them per round with
      // all their loads issued before any is written (one memory round trip per
      // round, not per pair: the compute waves wait for this at a GEMV's start)
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(d.X), 0, M * G * 64, kRsrcFlags);
      uint4* xs = reinterpret_cast<uint4*>(lds + d.xoff);
      for (int e0 = 0; e0 < 8 * G; e0 += 64 * kXRounds) {
        uint4 v[kXRounds][4];
#pragma unroll
        for (int u = 0; u < kXRounds; ++u) {
          const int e = e0 + 64 * u + lane, g = e >> 3, m = e & 7;
          const bool ok = e < 8 * G && m < M;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // an entry past X points past the resource: zeros, no access
            const int off = ok ? ((m * G + g) * 4 + c) * 16 : 0x7FFFFFF0;
            const u32x4_g tv = coherent
                                   ? __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kCoherent)
                                   : __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
            v[u][c] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
          }
        }
#pragma unroll
        for (int u = 0; u < kXRounds; ++u) {
          const int e = e0 + 64 * u + lane, g = e >> 3, m = e & 7;
          if (e < 8 * G && m < M) {
#pragma unroll
            for (int c = 0; c < 4; ++c) xs[(g * 4 + c) * 8 + m] = pair_order(v[u][c]);
          }
        }
      }
      wait_lds();
      if (lane == 0) lds_store(&sh.x_ready[(k - j0) % kSlots], k);
    }
    finish_upto(j1, true);
    if (me == 0) {
      for (unsigned it = 0; j0 <= j1 && !complete(j1); ++it) {
        if (it > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(8);
      }
      if (lane == 0) {
        const int e = lds_load(&sh.err);
        if (e) report_error(ctl, kErrX, e - 1);
      }
    }
  } else {
    // ---------------------------------------------------------- compute waves
    const int cw = wave - kSync;
    const int c = lane >> 4, r = lane & 15;
    // nibble masks (VGPR) and exponents (SGPR) of the pair decode, then the
    // offsets -1031 and -71 as fp16 pairs (SGPR)
    uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, e_lo = 0x64006400u, e_hi = 0x54005400u;
    uint32_t z_lo = 0xE407E407u, z_hi = 0xD470D470u;
    asm volatile("" : "+v"(m_lo), "+v"(m_hi));
    asm volatile("" : "+s"(e_lo), "+s"(e_hi));
    asm volatile("" : "+s"(z_lo), "+s"(z_hi));
    struct Cursor {
      TileDesc d;
      int j, t, t_end, row0;     // GEMV, next tile, end tile, first row of the workgroup
      int rows;                  // rows of the workgroup's y buffer for the GEMV
    } cu;
    // Spread mode deals a GEMV's tiles round-robin (a fixed deal: in a chain every
    // GEMV waits for its slowest wave, and claiming lets one wave take several
    // tiles of a short GEMV in a row).  Range mode: a wave claims its next tile of
    // the workgroup's stretch from an LDS counter when it starts a tile, so a wave
    // whose loads come back sooner takes more, and the waves run out of tiles
    // within about one tile of each other.  Either way a wave's tiles come in list
    // order, so its cursor only moves forward.
    int base = 0;
    auto enter = [&](int j) {
      for (; j <= j1; ++j) {
        const TileDesc d = read_desc(D + j);
        int t0, t1;
        tile_range(d.tbase, d.trem, d.N, t0, t1);
        int off = cw - base;
        if (off < 0) off += kCompute;
        base = (base + (t1 - t0)) % kCompute;
        if (t0 + off < t1) {
          cu.d = d;
          cu.j = j;
          cu.t = t0 + off;
          cu.t_end = t1;
          cu.row0 = t0 * 16;
          cu.rows = (t1 - t0) * 16;
          return;
        }
      }
      cu.j = j1 + 1;
    };
    // range mode: the cursor to tile T of the stretch (T >= the current tile)
    auto seek = [&](int T) {
      if (T >= rb) {
        cu.j = j1 + 1;
        return;
      }
      for (int j = cu.j; j <= j1; ++j) {
        const TileDesc d = j == cu.j ? cu.d : read_desc(D + j);
        if (T < d.tbase + (d.N + 15) / 16) {
          int t0, t1;
          tile_range(d.tbase, d.trem, d.N, t0, t1);
          cu.d = d;
          cu.j = j;
          cu.t = T - d.tbase;
          cu.t_end = t1;
          cu.row0 = t0 * 16;
          cu.rows = (t1 - t0) * 16;
          return;
        }
      }
      cu.j = j1 + 1;
    };
    const bool claiming = ranges != nullptr;
    auto claim_next = [&]() {
      int T = 0;
      if (lane == 0)
        T = __hip_atomic_fetch_add(&sh.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      seek(ra + __builtin_amdgcn_readfirstlane(T));
    };
    if (claiming) {
      cu.j = j0;
      if (j0 <= j1) {
        cu.d = read_desc(D + j0);
        claim_next();
      }
    } else {
      enter(j0);
    }
    auto wait_x = [&](int j) {
      for (unsigned it = 0; lds_load(&sh.x_ready[(j - j0) % kSlots]) != j; ++it) {
        if (it > kSpinLimit) {
          lds_store(&sh.err, j + 1);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    int cur = j0;
    auto signal_upto = [&](int j) {
      for (; cur < j; ++cur) {
        wait_x(cur);
        wait_lds();
        if (lane == 0) __hip_atomic_fetch_add(&sh.local_done[(cur - j0) % kSlots], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };

    // G % 8 == 0 and 16-byte aligned scales, and the stages were planned: the
    // staged path below
    auto staged = [&](const TileDesc& t) {
      return stage_off >= 0 && t.G % 8 == 0 && (reinterpret_cast<uintptr_t>(t.S) & 15u) == 0;
    };
    // A staged burst in flight: sixteen groups of the tile's 16 rows as four raw
    // loads of 8 rows x 128 contiguous bytes (w[2e + h]: groups 8e .. 8e + 7 of
    // the burst, rows 8h .. 8h + 7; lane l holds row 8h + l / 8, group l % 8), and
    // lane (c, r)'s row r scales of the two halves (s[e]).
    struct Pre {
      bool live;
      uint4 w[4];
      u32x4_g s[2];
    } pre;
    pre.live = false;
    auto issue_st = [&](Pre& P, const TileDesc& t, int tl, int b) {
      const int tr = tl * 16;
      const uint64_t left = (uint64_t)(t.N - tr) * (uint64_t)t.G;
      const uint32_t nw = left * 16 < 0xFFFFFFF0ull ? (uint32_t)(left * 16) : 0xFFFFFFF0u;
      const uint32_t ns = left * 2 < 0xFFFFFFF0ull ? (uint32_t)(left * 2) : 0xFFFFFFF0u;
      const __amdgpu_buffer_rsrc_t bw = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>((const uint4*)(t.W + (int64_t)tr * t.G)), 0, (int)nw, kRsrcFlags);
      const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((const uint16_t*)(t.S + (int64_t)tr * t.G)), 0, (int)ns,
          kRsrcFlags);
      // Only the per-lane offset is range-checked: rows past the matrix read zero
      // at every offset within the row, and a half past the row (G % 16 == 8, the
      // last burst) points past the resource (2 GiB - 16: out of range unless more
      // than 2 GiB follow, and then inside the matrix; never used).
      const bool two = 16 * b + 8 < t.G;
      // the scales first: they arrive last otherwise, and every burst waits for them
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int vs = e == 0 || two ? (r * t.G + 16 * b + 8 * e) * 2 : 0x7FFFFFF0;
        P.s[e] = __builtin_amdgcn_raw_buffer_load_b128(bs, vs, 0, 0);
      }
      const int vo = ((lane >> 3) * t.G + (lane & 7)) * 16;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int so = __builtin_amdgcn_readfirstlane((16 * b + 8 * e) * 16);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int v = e == 0 || two ? vo + h * 128 * t.G : 0x7FFFFFF0;
          const u32x4_g a = __builtin_amdgcn_raw_buffer_load_b128(bw, v, so, kNonTemporal);
          P.w[2 * e + h] = make_uint4(a[0], a[1], a[2], a[3]);
        }
      }
      P.live = true;
    };
    while (cu.j <= j1) {
      const TileDesc d = cu.d;
      const int j = cu.j, G = d.G, tile = cu.t;
      const int tr0 = tile * 16;                      // first row of the tile
      const uint64_t left = (uint64_t)(d.N - tr0) * (uint64_t)G;
      const uint32_t nw = left * 16 < 0xFFFFFFF0ull ? (uint32_t)(left * 16) : 0xFFFFFFF0u;
      const uint32_t ns = left * 2 < 0xFFFFFFF0ull ? (uint32_t)(left * 2) : 0xFFFFFFF0u;
      const __amdgpu_buffer_rsrc_t bw = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>((const uint4*)(d.W + (int64_t)tr0 * G)), 0, (int)nw, kRsrcFlags);
      const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((const uint16_t*)(d.S + (int64_t)tr0 * G)), 0, (int)ns,
          kRsrcFlags);
      // rows past the matrix end read zero: only the per-lane offset is range-checked,
      // and a row past the end is past the end at every chunk
      const int vo_w = (r * G + c) * 16, vo_s = r * G * 2;
      const int nch = G / 4;
      const bool wide = staged(d);
      const int xo = d.xoff;
      const int rows = cu.rows;
      const int wrow0 = cu.row0;
      // advance the cursor before the loads are consumed
      if (claiming) {
        claim_next();
      } else {
        cu.t += kCompute;
        if (cu.t >= cu.t_end) enter(cu.j + 1);
      }

      f4_t acc = {0.f, 0.f, 0.f, 0.f};
      // Lane (c, r) supplies row r of A (X) and receives rows 4c..4c+3 of D.  Rows
      // of X past M and the lanes with c >= 2 only feed rows of D that are never
      // stored, so they read row M - 1 instead of zeros: every lane reads valid
      // LDS without a branch.  Per group the addresses advance by a fixed stride
      // from a per-lane base.
      const uint8_t* a_base = lds + xo + (c * 8 + (r < M ? r : M - 1)) * 16;
      constexpr int a_step = 512;                     // X planes: bytes per group
      auto x_of = [&](int g) { return *reinterpret_cast<const uint4*>(a_base + g * a_step); };
      // two codes as the exact fp16 pair (q - 7, q' - 7)
      auto dq = [&](uint32_t t, uint32_t m, uint32_t e, uint32_t z) {
        return bits<uint32_t>(bits<h2_t>((t & m) | e) + bits<h2_t>(z));
      };
      // one group of the tile: B from word c of the group in lane (c, r), A = X rows
      const f4_t zero4 = {0.f, 0.f, 0.f, 0.f};
      auto group_mma = [&](uint32_t vt, uint4 a) {
        const uint32_t x8 = vt >> 8;
        const uint4 bq = make_uint4(dq(vt, m_lo, e_lo, z_lo), dq(vt, m_hi, e_hi, z_hi),
                                    dq(x8, m_lo, e_lo, z_lo), dq(x8, m_hi, e_hi, z_hi));
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(bits<h8_t>(a), bits<h8_t>(bq), zero4, 0, 0,
                                                      0);
      };
      // the group's scale, applied exactly in fp32
      auto scale_add = [&](f4_t dd, uint32_t sbits) {
        const float sv = (float)bits<_Float16>((uint16_t)sbits);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sv, dd[e], acc[e]);
      };
      if (wide) {
        // Bursts of sixteen groups of the tile's 16 rows, loaded as instructions of
        // 8 rows x 128 contiguous bytes (lane l: row 8h + l / 8, group l % 8), so
        // each touches 8 whole cache lines -- not 16 half lines, which streams at
        // two thirds of the rate.  Each half (eight groups) goes through this
        // wave's LDS stage as word planes [word][16 rows][8 groups] of dwords, so
        // lane (c, r) reads word c of the eight groups of row r as 32 contiguous
        // bytes: B's layout, with no exchange between lanes.  Once the raw
        // registers are in LDS, the next burst (of this tile, or the first of the
        // next one) is issued, so loads stay in flight while a burst is computed.
        const int nb = (G + 15) / 16;
        if (!pre.live) issue_st(pre, d, tile, 0);
        uint32_t* const st = reinterpret_cast<uint32_t*>(lds + stage_off + cw * kStage);
        const uint4* const sr = reinterpret_cast<const uint4*>(st + c * 128 + r * 8);
        for (int b = 0; b < nb; ++b) {
          const bool two = 16 * b + 8 < G;
          const u32x4_g sc0 = pre.s[0], sc1 = pre.s[1];
          uint4 wq[2][2];                       // [half][groups 0-3, 4-7]: word c, row r
          auto stage_half = [&](const uint4& lo, const uint4& hi) {
            st[0 * 128 + lane] = lo.x;          // plane w: [row][group] dwords
            st[1 * 128 + lane] = lo.y;
            st[2 * 128 + lane] = lo.z;
            st[3 * 128 + lane] = lo.w;
            st[0 * 128 + 64 + lane] = hi.x;     // rows 8..15
            st[1 * 128 + 64 + lane] = hi.y;
            st[2 * 128 + 64 + lane] = hi.z;
            st[3 * 128 + 64 + lane] = hi.w;
          };
          stage_half(pre.w[0], pre.w[1]);
          wq[0][0] = sr[0];
          wq[0][1] = sr[1];
          if (two) {                            // the stage is reused in order
            stage_half(pre.w[2], pre.w[3]);
            wq[1][0] = sr[0];
            wq[1][1] = sr[1];
          }
          if (b + 1 < nb) {
            issue_st(pre, d, tile, b + 1);
          } else if (cu.j <= j1 && staged(cu.d)) {
            issue_st(pre, cu.d, cu.t, 0);
          } else {
            pre.live = false;
          }
          if (b == 0) {
            signal_upto(j);
            wait_x(j);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if (e == 1 && !two) break;
            const int g0 = 16 * b + 8 * e;
            const u32x4_g sc = e == 0 ? sc0 : sc1;
            // X of the half's groups: one address, immediate offsets
            const uint8_t* const ab = a_base + g0 * a_step;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint4 w4 = wq[e][h];
              const uint32_t v[4] = {w4.x, w4.y, w4.z, w4.w};   // word c of group g0 + 4h + t
              uint4 xa[4];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                xa[t] = *reinterpret_cast<const uint4*>(ab + (4 * h + t) * a_step);
#pragma unroll
              for (int t = 0; t < 4; t += 2) {
                const uint32_t sw = sc[2 * h + t / 2];   // scales of groups g0 + 4h + t, + t + 1
                const f4_t d0 = group_mma(v[t], xa[t]);
                const f4_t d1 = group_mma(v[t + 1], xa[t + 1]);
                scale_add(d0, sw & 0xFFFFu);
                scale_add(d1, sw >> 16);
              }
            }
          }
        }
      } else {
        for (int ch0 = 0; ch0 < nch; ch0 += kChunks) {
          uint4 w[kChunks];
          u32x2_g s[kChunks];
#pragma unroll
          for (int q = 0; q < kChunks; ++q) {
            const int ch = ch0 + q < nch ? ch0 + q : nch - 1;   // past the row: re-read
            const int so = __builtin_amdgcn_readfirstlane(ch);
            const u32x4_g v = __builtin_amdgcn_raw_buffer_load_b128(bw, vo_w, so * 64, kNonTemporal);
            w[q] = make_uint4(v[0], v[1], v[2], v[3]);
            s[q] = __builtin_amdgcn_raw_buffer_load_b64(bs, vo_s, so * 8, 0);
          }
          if (ch0 == 0) {
            signal_upto(j);
            wait_x(j);
          }
#pragma unroll
          for (int q = 0; q < kChunks; ++q) {
            if (ch0 + q < nch) {
              const int g0 = (ch0 + q) * 4;
              uint4 xa[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) xa[t] = x_of(g0 + t);
              uint32_t v[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
              transpose4(v);                    // v[t]: word c of group g0 + t, row r
              const uint32_t sc[4] = {s[q][0] & 0xFFFFu, s[q][0] >> 16, s[q][1] & 0xFFFFu,
                                      s[q][1] >> 16};
#pragma unroll
              for (int t = 0; t < 4; t += 2) {
                const f4_t d0 = group_mma(v[t], xa[t]);
                const f4_t d1 = group_mma(v[t + 1], xa[t + 1]);
                scale_add(d0, sc[t]);
                scale_add(d1, sc[t + 1]);
              }
            }
          }
        }
      }
      // lane (c, r) holds rows m = 4c + e of column n = tr0 + r
      if (c < 2 && tr0 + r < d.N) {
        uint16_t* yb = reinterpret_cast<uint16_t*>(lds + xo + ybuf_off(M, G));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 4 * c + e;
          if (m < M) yb[m * rows + (tr0 + r - wrow0)] = bits<uint16_t>((_Float16)acc[e]);
        }
      }
    }
    signal_upto(j1 + 1);
  }

  // leave the counters zeroed for the next call (the last workgroup clears them)
  __syncthreads();
  if (wave == 0) {
    unsigned old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(ctl + kCtlExit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == (unsigned)nwg - 1u) {
      for (int i = lane; i < n; i += 64)
        __hip_atomic_store(done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(ctl + kCtlExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

MStepPlan plan_step_mfma(const DeviceInfo& dev, const StepLayer* layers, int64_t n, int M,
                         bool ordered) {
  MStepPlan p;
  if (n < 1 || M < 2 || M > 8) return p;
  p.grid = dev.cus;
  p.M = M;
  p.desc.resize((size_t)n);
  std::vector<int64_t> tiles((size_t)n);
  for (int64_t k = 0; k < n; ++k) {
    const StepLayer& L = layers[k];
    if (L.K % 128 || L.K > 8192 || L.N >= (1 << 24) || L.x_op) return p;
    if (reinterpret_cast<uintptr_t>(L.scales) % 8) return p;   // 8-byte scale loads
    MStepDesc& s = p.desc[(size_t)k];
    s.W = reinterpret_cast<const uint4*>(L.words);
    s.S = L.scales;
    s.X = reinterpret_cast<const uint4*>(L.x);
    s.Y = L.y;
    s.N = (int)L.N;
    s.G = (int)(L.K / 32);
    s.dep = -1;
    s.signal = 0;
    s.rel = -1;
    tiles[(size_t)k] = (L.N + 15) / 16;
  }
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
  };
  // k waits for its latest conflict (an earlier GEMV writing what k reads or
  // writes, or reading what k writes; ordered: also k - 1).  A workgroup publishes
  // a GEMV only after staging the X of every GEMV before it, and stages X only
  // after its own wait, so the wait also covers every writer reached from it
  // through waits (and every reader before it); a list with a writer not covered
  // so runs one kernel per GEMV.
  for (int64_t k = 1; k < n; ++k) {
    int dep = ordered ? (int)k - 1 : -1;
    std::vector<int> writers;
    const StepLayer& Lk = layers[k];
    for (int64_t i = k - 1; i >= 0; --i) {
      const StepLayer& Li = layers[i];
      const int64_t yi = 2 * M * Li.N, xk = 2 * M * Lk.K, yk = 2 * M * Lk.N;
      const bool w = overlap(Li.y, yi, Lk.x, xk) || overlap(Li.y, yi, Lk.y, yk);
      if (w) writers.push_back((int)i);
      if ((w || overlap(Li.x, 2 * M * Li.K, Lk.y, yk)) && (int)i > dep) dep = (int)i;
    }
    p.desc[(size_t)k].dep = dep;
    if (dep >= 0) {
      p.desc[(size_t)dep].signal = 1;
      p.cross_wg = true;
    }
    for (int h : writers) {
      int i = dep;
      while (i > h && p.desc[(size_t)i].dep >= 0) i = p.desc[(size_t)i].dep;
      if (i != h) return p;                     // not covered: one kernel per GEMV
    }
  }
  // static LDS and margin, then the compute waves' stages at the end; the X
  // regions share the rest.  A list whose regions do not fit beside the stages
  // goes without them (stage_off < 0: every GEMV takes the unstaged path).
  const size_t total_lds = (size_t)dev.lds_per_block - 1024;
  size_t cap = total_lds - (size_t)kCompute * kStage;
  p.stage_off = (int)cap;
  // the most rows any workgroup holds of each GEMV, per mode
  std::vector<int64_t> rows((size_t)n);
  // LDS regions as a ring in list order; rel: the latest earlier user of the space
  auto place_in = [&]() {
    std::vector<size_t> off((size_t)n), size((size_t)n);
    size_t cur = 0;
    for (int64_t k = 0; k < n; ++k) {
      MStepDesc& s = p.desc[(size_t)k];
      const size_t sz = (size_t)8 * s.G * 64 +
                        (((size_t)rows[(size_t)k] * M * 2 + 15) & ~(size_t)15);
      if (sz > cap) return false;
      if (cur + sz > cap) cur = 0;
      off[(size_t)k] = cur;
      size[(size_t)k] = sz;
      s.xoff = (int)cur;
      cur += sz;
      s.rel = -1;
      for (int64_t i = k - 1; i >= 0; --i) {
        if (off[(size_t)i] < cur && cur - sz < off[(size_t)i] + size[(size_t)i]) {
          s.rel = (int)i;
          break;
        }
      }
    }
    return true;
  };
  // without the stages if the regions do not fit beside them
  auto place = [&]() {
    if (place_in()) return true;
    if (p.stage_off < 0) return false;
    p.stage_off = -1;
    cap = total_lds;
    return place_in();
  };
  // Range mode (no dependencies): each workgroup takes one contiguous stretch of
  // the 16-row tiles of all GEMVs laid end to end, balanced by weight bytes and
  // the GEMV boundaries inside each stretch (kBoundaryCost).
  if (!p.cross_wg) {
    std::vector<int64_t> first((size_t)n + 1), cum((size_t)n + 1);
    for (int64_t k = 0; k < n; ++k) {
      const int64_t tb = 16 * (int64_t)p.desc[(size_t)k].G * 18;
      first[(size_t)k + 1] = first[(size_t)k] + tiles[(size_t)k];
      cum[(size_t)k + 1] = cum[(size_t)k] + tb * tiles[(size_t)k];
    }
    const int64_t total = cum[(size_t)n];
    std::vector<int64_t> cut((size_t)p.grid + 1);
    // Stretches of least maximum cost, where a stretch costs its bytes plus
    // kBoundaryCost for every GEMV it starts after its first one: greedy filling
    // under a budget, the budget found by bisection.
    // (A GEMV's tiles all cost the same, so a stretch takes them in runs: the
    // host work is per GEMV and stretch, not per tile.)
    auto fill = [&](int64_t budget, bool keep) {
      int w = 0;
      int64_t used = 0;
      if (keep) cut[0] = 0;
      for (int64_t k = 0; k < n; ++k) {
        const int64_t tb = 16 * (int64_t)p.desc[(size_t)k].G * 18, nt = tiles[(size_t)k];
        for (int64_t t = 0; t < nt;) {
          const int64_t c = tb + (t == 0 && used > 0 ? kBoundaryCost : 0);
          if (used + c > budget && used > 0) {   // the next stretch starts at tile t
            if (++w >= p.grid) return false;
            if (keep) cut[(size_t)w] = first[(size_t)k] + t;
            used = 0;
            continue;
          }
          used += c;                             // this tile, then all that still fit
          ++t;
          const int64_t more = std::min<int64_t>(nt - t, (budget - used) / tb);
          if (more > 0) {
            used += more * tb;
            t += more;
          }
        }
      }
      if (keep)
        for (int v = w + 1; v <= p.grid; ++v) cut[(size_t)v] = first[(size_t)n];
      return true;
    };
    int64_t lo = (total + p.grid - 1) / p.grid, hi = lo;
    while (!fill(hi, false)) hi *= 2;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (fill(mid, false)) hi = mid; else lo = mid + 1;
    }
    fill(hi, true);
    auto gemv_of = [&](int64_t t) {
      return (int)(std::upper_bound(first.begin(), first.end(), t) - first.begin() - 1);
    };
    std::vector<int> ranges((size_t)p.grid * 4);
    std::fill(rows.begin(), rows.end(), 16);
    for (int w = 0; w < p.grid; ++w) {
      const int64_t a = cut[(size_t)w], b = cut[(size_t)w + 1];
      int j0 = 1, j1 = 0;
      if (b > a) {
        j0 = gemv_of(a);
        j1 = gemv_of(b - 1);
        for (int j = j0; j <= j1; ++j) {
          const int64_t lo = std::max<int64_t>(a - first[(size_t)j], 0);
          const int64_t hi = std::min<int64_t>(b - first[(size_t)j], tiles[(size_t)j]);
          rows[(size_t)j] = std::max<int64_t>(rows[(size_t)j], (hi - lo) * 16);
        }
      }
      ranges[(size_t)w * 4 + 0] = (int)a;
      ranges[(size_t)w * 4 + 1] = (int)b;
      ranges[(size_t)w * 4 + 2] = j0;
      ranges[(size_t)w * 4 + 3] = j1;
    }
    if (first[(size_t)n] < INT32_MAX && place()) {
      for (int64_t k = 0; k < n; ++k) {
        p.desc[(size_t)k].tbase = (int)first[(size_t)k];
        p.desc[(size_t)k].trem = -1;
      }
      p.ranges = std::move(ranges);
      p.lds_bytes = total_lds;
      p.ok = true;
      return p;
    }
  }
  for (int64_t k = 0; k < n; ++k) {
    MStepDesc& s = p.desc[(size_t)k];
    s.tbase = (int)(tiles[(size_t)k] / p.grid);
    s.trem = (int)(tiles[(size_t)k] % p.grid);
    rows[(size_t)k] = (int64_t)(s.tbase + (s.trem > 0)) * 16;
  }
  if (!place()) return p;
  p.lds_bytes = total_lds;
  p.ok = true;
  return p;
}

StepLaunch step_mfma_launch_of(const MStepPlan& p) {
  StepLaunch L{};
  L.kind = 2;
  L.n = (int)p.desc.size();
  L.grid = p.grid;
  L.M = p.M;
  L.stage_off = p.stage_off;
  L.cross_wg = p.cross_wg;
  L.has_ranges = !p.ranges.empty();
  L.lds_bytes = (uint32_t)p.lds_bytes;
  L.clear_bytes = (((uint64_t)kCtlWords + p.desc.size()) * 4 + 255) & ~(uint64_t)255;
  L.table_off = L.clear_bytes;
  L.ranges_off = L.table_off + p.desc.size() * sizeof(MStepDesc);
  L.table_bytes = p.desc.size() * sizeof(MStepDesc) + p.ranges.size() * sizeof(int);
  L.ws_bytes = L.table_off + L.table_bytes;
  return L;
}

void step_mfma_table_bytes(const MStepPlan& p, std::vector<uint8_t>* out) {
  const size_t db = p.desc.size() * sizeof(MStepDesc);
  out->resize(db + p.ranges.size() * sizeof(int));
  std::memcpy(out->data(), p.desc.data(), db);
  if (!p.ranges.empty())
    std::memcpy(out->data() + db, p.ranges.data(), p.ranges.size() * sizeof(int));
}

hipError_t step_mfma_occupancy(const MStepPlan& p, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, reinterpret_cast<const void*>(k_step_mfma), kStepThreads, p.lds_bytes);
}

hipError_t step_mfma_prepare(const StepLaunch& L) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k_step_mfma),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds_bytes);
}

hipError_t launch_step_mfma(const StepLaunch& L, void* ws, hipStream_t s) {
  unsigned* ctl = static_cast<unsigned*>(ws);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const MStepDesc* desc = reinterpret_cast<const MStepDesc*>(base + L.table_off);
  const int4* rg = L.has_ranges ? reinterpret_cast<const int4*>(base + L.ranges_off) : nullptr;
  int n = L.n, M = L.M, so = L.stage_off;
  if (L.cross_wg) {
    void* args[] = {(void*)&desc, (void*)&n, (void*)&M, (void*)&ctl, (void*)&rg, (void*)&so};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_step_mfma), dim3(L.grid),
                                      dim3(kStepThreads), args, L.lds_bytes, s);
  }
  hipLaunchKernelGGL(k_step_mfma, dim3(L.grid), dim3(kStepThreads), L.lds_bytes, s, desc, n, M,
                     ctl, rg, so);
  return hipGetLastError();
}

}  // namespace q4
