// Persistent decode-step kernel, LDS-ring variant: the weight stream goes from
// HBM straight into LDS by asynchronous DMA, so prefetch depth costs LDS instead
// of registers.
//
// One workgroup of 16 waves per compute unit (cooperative launch):
//  * kLoaders loader waves: walk this workgroup's tiles -- up to 12 KB of
//    consecutive rows of one GEMV -- in list order, loader l taking every
//    kLoaders-th tile, and copy each tile's packed words and fp16 scales into an
//    LDS ring slot with global_load_lds_dwordx4 (1 KB per instruction, 16 bytes
//    per lane, like a plain streaming read).  A tile is marked full once the
//    in-order vector-memory counter shows its copies have landed.  One wave alone
//    cannot issue copies fast enough to keep HBM busy; one per SIMD can.
//  * waves 0 .. kSync-1 (sync): as in the register variant -- stage x of their
//    GEMVs into LDS (pair-ordered planes plus per-group bias terms), copy finished
//    y rows out, publish per-GEMV completion for dependent GEMVs.
//  * the other waves (compute): take full tiles in order from a shared counter,
//    read words, scales and x from LDS, process the tile's row-steps two at a
//    time (one read of x serves both) and write y rows to LDS.
//
// Requirements (checked on the host): every K is a multiple of 256 and at most
// 8192, scales are 16-byte aligned.  Then a row's words (K/2 bytes) and scales
// (K/16 bytes) are whole 16-byte chunks, and 2^lpr lanes x C groups cover a row
// exactly (C <= 8).
#include "q4_step_dma.h"

namespace q4 {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));
#define Q4_GLOBAL __attribute__((address_space(1)))

template <typename T, typename F>
__device__ __forceinline__ T bits(F v) {
  return __builtin_bit_cast(T, v);
}

__device__ __forceinline__ uint4 pair_order(uint4 v) {
  uint4 o;
  o.x = (v.x & 0xFFFFu) | (v.z << 16);
  o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
  o.z = (v.y & 0xFFFFu) | (v.w << 16);
  o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
  return o;
}

// Nibble-pair constants: masks in VGPRs, exponents in SGPRs, so each pair is one
// v_and_or_b32 (see the register variant for the derivation).
struct Nibbles {
  uint32_t m_lo, m_hi, e_lo, e_hi;
};
__device__ __forceinline__ Nibbles make_nibbles() {
  Nibbles n{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
  asm volatile("" : "+v"(n.m_lo), "+v"(n.m_hi));
  asm volatile("" : "+s"(n.e_lo), "+s"(n.e_hi));
  return n;
}

// sum over one group of (q - 7) x, the chain seeded with minus the group's bias
__device__ __forceinline__ float group_dot(uint4 w, const uint4 (&x)[4], float neg_bias,
                                          const Nibbles& nb) {
  const uint32_t wj[4] = {w.x, w.y, w.z, w.w};
  float a = neg_bias, b = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = wj[j], v8 = v >> 8;
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v & nb.m_lo) | nb.e_lo), bits<h2_t>(x[j].x), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v & nb.m_hi) | nb.e_hi), bits<h2_t>(x[j].y), b, false);
    a = __builtin_amdgcn_fdot2(bits<h2_t>((v8 & nb.m_lo) | nb.e_lo), bits<h2_t>(x[j].z), a, false);
    b = __builtin_amdgcn_fdot2(bits<h2_t>((v8 & nb.m_hi) | nb.e_hi), bits<h2_t>(x[j].w), b, false);
  }
  return a + b;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return bits<float>(__builtin_amdgcn_update_dpp(0, bits<int>(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float team_sum(float v, int lg) {
  if (lg >= 1) v += dpp<0xB1>(v);
  if (lg >= 2) v += dpp<0x4E>(v);
  if (lg >= 3) v += dpp<0x141>(v);
  if (lg >= 4) v += dpp<0x140>(v);
  if (lg >= 5) {
    const auto r = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  if (lg >= 6) {
    const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(v), bits<uint32_t>(v),
                                                    false, false);
    v = bits<float>((uint32_t)r[0]) + bits<float>((uint32_t)r[1]);
  }
  return v;
}

__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The loaders move tiles with plain 16-byte-per-lane loads into registers (the
// same access as a streaming read) and 16-byte LDS writes, two register tiles
// alternating.  One step is a single inline-assembly block: issue the nine loads
// of the next tile into one register set, wait until only those nine are
// outstanding (the vector-memory counter drains in order, so the previous tile
// has landed), write the previous tile from the other set to its LDS slot, and
// wait for the writes.  The compiler sees both sets as read and written by every
// step, so it never copies or reuses them while loads are in flight, and it
// inserts no waits of its own (it would drain every load before each write).
// Loader waves issue no other vector-memory instruction.
typedef const Q4_GLOBAL uint8_t* gaddr_t;
constexpr int kTileLoads = 9;                     // 8 x 1 KB of words + 1 KB of scales

#define Q4_TILE_LOADS(R, A)                                      \
  "global_load_dwordx4 %[" #R "0], %[" #A "0], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "1], %[" #A "1], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "2], %[" #A "2], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "3], %[" #A "3], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "4], %[" #A "4], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "5], %[" #A "5], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "6], %[" #A "6], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "7], %[" #A "7], off nt\n\t"       \
  "global_load_dwordx4 %[" #R "8], %[" #A "8], off nt\n\t"
#define Q4_TILE_WRITES(R)                                        \
  "ds_write_b128 %[l], %[" #R "0]\n\t"                           \
  "ds_write_b128 %[l], %[" #R "1] offset:1024\n\t"               \
  "ds_write_b128 %[l], %[" #R "2] offset:2048\n\t"               \
  "ds_write_b128 %[l], %[" #R "3] offset:3072\n\t"               \
  "ds_write_b128 %[l], %[" #R "4] offset:4096\n\t"               \
  "ds_write_b128 %[l], %[" #R "5] offset:5120\n\t"               \
  "ds_write_b128 %[l], %[" #R "6] offset:6144\n\t"               \
  "ds_write_b128 %[l], %[" #R "7] offset:7168\n\t"               \
  "ds_write_b128 %[l], %[" #R "8] offset:8192\n\t"
#define Q4_REGS(N, R)                                                                   \
  [N##0] "+v"(R[0]), [N##1] "+v"(R[1]), [N##2] "+v"(R[2]), [N##3] "+v"(R[3]),           \
      [N##4] "+v"(R[4]), [N##5] "+v"(R[5]), [N##6] "+v"(R[6]), [N##7] "+v"(R[7]),       \
      [N##8] "+v"(R[8])
#define Q4_ADDRS(A)                                                                     \
  [a0] "v"(A[0]), [a1] "v"(A[1]), [a2] "v"(A[2]), [a3] "v"(A[3]), [a4] "v"(A[4]),       \
      [a5] "v"(A[5]), [a6] "v"(A[6]), [a7] "v"(A[7]), [a8] "v"(A[8])

// issue the loads of a tile into nx
__device__ __forceinline__ void tile_issue(u32x4_g (&nx)[kTileLoads], u32x4_g (&other)[kTileLoads],
                                           const gaddr_t (&a)[kTileLoads]) {
  asm volatile(Q4_TILE_LOADS(n, a) "" : Q4_REGS(n, nx), Q4_REGS(c, other) : Q4_ADDRS(a) : "memory");
}
// issue the loads of the next tile into nx, then write cur (loaded before) to LDS
__device__ __forceinline__ void tile_step(u32x4_g (&nx)[kTileLoads], u32x4_g (&cur)[kTileLoads],
                                          const gaddr_t (&a)[kTileLoads], uint32_t lds) {
  asm volatile(Q4_TILE_LOADS(n, a) "s_waitcnt vmcnt(9)\n\t" Q4_TILE_WRITES(c) "s_waitcnt lgkmcnt(0)"
               : Q4_REGS(n, nx), Q4_REGS(c, cur)
               : Q4_ADDRS(a), [l] "v"(lds)
               : "memory");
}
// wait for every load (the last, never written tile)
__device__ __forceinline__ void tile_drain(u32x4_g (&x)[kTileLoads], u32x4_g (&y)[kTileLoads]) {
  asm volatile("s_waitcnt vmcnt(0)" : Q4_REGS(n, x), Q4_REGS(c, y) : : "memory");
}

// What a loader needs of a descriptor, read with scalar loads issued as inline
// assembly: ordinary loads after the assembly above may not be proven unchanged,
// so the compiler would make them vector loads and drain the whole tile stream
// (vmcnt(0)) before using them.
struct LoaderDesc {
  const Q4_GLOBAL uint8_t* W;
  const Q4_GLOBAL uint8_t* S;
  int N, G, tr, tiles;
};
typedef uint32_t u32x2_s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ LoaderDesc read_desc(const DmaDesc* d) {
  u32x4_g ws;
  u32x2_s ng, tt;
  asm volatile(
      "s_load_dwordx4 %0, %3, 0x0\n\t"
      "s_load_dwordx2 %1, %3, 0x20\n\t"
      "s_load_dwordx2 %2, %3, 0x30\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(ws), "=&s"(ng), "=&s"(tt)
      : "s"(d));
  static_assert(offsetof(DmaDesc, S) == 8 && offsetof(DmaDesc, N) == 32 &&
                    offsetof(DmaDesc, G) == 36 && offsetof(DmaDesc, tr) == 48 &&
                    offsetof(DmaDesc, tiles) == 52,
                "descriptor offsets read by the loaders");
  LoaderDesc r;
  r.W = (const Q4_GLOBAL uint8_t*)(((uint64_t)ws[1] << 32) | ws[0]);
  r.S = (const Q4_GLOBAL uint8_t*)(((uint64_t)ws[3] << 32) | ws[2]);
  r.N = (int)ng[0];
  r.G = (int)ng[1];
  r.tr = (int)tt[0];
  r.tiles = (int)tt[1];
  return r;
}

constexpr int kWaves = kStepThreads / 64;        // 16
constexpr int kSync = 2;                         // sync waves
constexpr int kLoader0 = kSync;                  // first loader wave
constexpr int kCompute = kWaves - kSync - kLoaders;   // compute waves
constexpr int kPerLoader = kSlots / kLoaders;    // slots (and tiles in flight) per loader
constexpr int kWordLoads = kSlotWordBytes / 1024;      // per lane and tile
constexpr int kScaleLoads = (kSlotWordBytes / 8 + 1023) / 1024;
constexpr unsigned kSpinLimit = 1u << 24;
constexpr int kCoherent = 1 | 16;                // sc0 | sc1
constexpr int kWaitVm0 = 0x0F70;                 // s_waitcnt vmcnt(0)
static_assert(kDmaXBufs % kSync == 0, "x-buffer owner");
static_assert(kSlots % kLoaders == 0 && kPerLoader >= 1, "slots per loader");
static_assert(kWordLoads == 8 && kScaleLoads == 1 && kWordLoads + kScaleLoads == kTileLoads,
              "the loader's register tiles");
static_assert(kScaleLoads * 1024 <= kSlotScaleBytes, "scale copies fit the slot");
static_assert(kCompute >= 4, "compute waves");

struct Shared {
  int x_ready[kDmaXBufs];     // GEMV whose x sits in buffer b (-1: none)
  int tiles_done[kDmaXBufs];  // tiles of that GEMV finished by compute waves
  int slot_tile[kSlots];      // tile whose copy into the slot has landed (-1: none)
  int slot_free[kSlots];      // last tile read out of the slot (-1: none)
  int slot_j[kSlots];         // GEMV, first row and rows of the tile in the slot
  int slot_row0[kSlots];
  int slot_rows[kSlots];
  int next_tile;              // tile counter for compute waves
  int err;
};

__device__ __forceinline__ int split(int total, int wg, int nwg) {
  return (int)(((unsigned)total * (unsigned)wg) / (unsigned)nwg);
}

__global__ __launch_bounds__(kStepThreads) void k_step_dma(const DmaDesc* __restrict__ D, int n,
                                                           unsigned* __restrict__ done,
                                                           unsigned* __restrict__ err,
                                                           int maxG, int ybuf_rows) {
  extern __shared__ uint4 smem[];
  __shared__ Shared sh;
  // LDS: [kSlots] x (8 KB words + 1 KB scales) | [NX] x 4 x maxG x 16 B x |
  //      [NX] x maxG floats bias | [NX] x ybuf_rows fp16 y
  uint4* ring = smem;
  uint4* xbuf = ring + kSlots * (kSlotBytes / 16);
  float* cbuf = reinterpret_cast<float*>(xbuf + kDmaXBufs * 4 * maxG);
  uint16_t* ybuf = reinterpret_cast<uint16_t*>(cbuf + kDmaXBufs * maxG);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x, nwg = gridDim.x;
  if (threadIdx.x < kDmaXBufs) {
    sh.x_ready[threadIdx.x] = -1;
    sh.tiles_done[threadIdx.x] = 0;
  }
  if (threadIdx.x < kSlots) {
    sh.slot_tile[threadIdx.x] = -1;
    sh.slot_free[threadIdx.x] = -1;
  }
  if (threadIdx.x == 0) {
    sh.next_tile = 0;
    sh.err = 0;
  }
  __syncthreads();

  if (wave >= kLoader0 && wave < kLoader0 + kLoaders) {
    // ---------------------------------------------------------------- loaders
    // Loader l moves tiles l, l + kLoaders, ... of this workgroup's tile list
    // (GEMVs in list order, each GEMV's tiles split evenly over workgroups) into
    // slots l, l + kLoaders, ...  Two register tiles alternate: the loads of the
    // next tile are issued before the current one is waited for and written to
    // its slot, so the stream does not stop while a slot is still being read.
    const int l = wave - kLoader0;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    int total = 0;
    for (int i = 0; i < n; ++i) total += split(D[i].tiles, wg + 1, nwg) - split(D[i].tiles, wg, nwg);
    const int mine = total > l ? (total - l + kLoaders - 1) / kLoaders : 0;
    int j = 0;
    LoaderDesc cd = read_desc(D);
    int tt = split(cd.tiles, wg, nwg), tend = split(cd.tiles, wg + 1, nwg);
    auto advance = [&](int by) {                 // move the cursor `by` tiles on
      tt += by;
      while (tt >= tend && j + 1 < n) {
        const int over = tt - tend;
        ++j;
        cd = read_desc(D + j);
        tt = split(cd.tiles, wg, nwg) + over;
        tend = split(cd.tiles, wg + 1, nwg);
      }
    };
    advance(l);
    struct Meta {                                // the tile a register set holds
      int j, row0, rows;
    };
    // the cursor's tile: its metadata and the nine per-lane addresses
    auto address = [&](Meta& m, gaddr_t (&a)[kTileLoads]) {
      const int wrow = cd.G * 16, srow = cd.G * 2;     // bytes per row: words, scales
      m.j = j;
      m.row0 = tt * cd.tr;
      m.rows = cd.N - m.row0 < cd.tr ? cd.N - m.row0 : cd.tr;
      const int wbytes = m.rows * wrow, sbytes = m.rows * srow;   // multiples of 16
      const gaddr_t wt = cd.W + (int64_t)m.row0 * wrow;
#pragma unroll
      for (int c = 0; c < kWordLoads; ++c) {
        int off = c * 1024 + lane * 16;
        if (off >= wbytes) off = wbytes - 16;       // past the tile: re-read its last chunk
        a[c] = wt + off;
      }
      int off = lane * 16;
      if (off >= sbytes) off = sbytes - 16;
      a[kWordLoads] = cd.S + (int64_t)m.row0 * srow + off;
    };
    auto claim = [&](const Meta& m, int i) {      // wait for tile i's slot; its header
      const int t = l + i * kLoaders;
      const int slot = t % kSlots;
      if (t >= kSlots) {
        for (unsigned it = 0; lds_load(&sh.slot_free[slot]) < t - kSlots; ++it) {
          if (it > kSpinLimit) { lds_store(&sh.err, 4); break; }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (lane == 0) {
        sh.slot_j[slot] = m.j;
        sh.slot_row0[slot] = m.row0;
        sh.slot_rows[slot] = m.rows;
      }
      return ring_lds + (uint32_t)slot * kSlotBytes + lane * 16;
    };
    auto publish = [&](int i) {
      const int t = l + i * kLoaders;
      if (lane == 0) lds_store(&sh.slot_tile[t % kSlots], t);
    };
    // Every step issues one tile's loads (after the last tile the cursor stays
    // put and its tile is read again, never written), so the in-flight count at
    // each wait is exactly one tile.
    if (mine > 0) {
      u32x4_g A[kTileLoads], B[kTileLoads];
      gaddr_t adr[kTileLoads];
      Meta mA, mB;
      int issued = 0;
      auto next = [&](Meta& m) {
        address(m, adr);
        if (++issued < mine) advance(kLoaders);
      };
      next(mA);
      tile_issue(A, B, adr);
      for (int i = 0;;) {
        next(mB);
        tile_step(B, A, adr, claim(mA, i));
        publish(i);
        if (++i == mine) break;
        next(mA);
        tile_step(A, B, adr, claim(mB, i));
        publish(i);
        if (++i == mine) break;
      }
      tile_drain(A, B);
    }
    return;
  }

  if (wave < kSync) {
    // ------------------------------------------------------------- sync waves
    const int me = wave;
    int next_fin = me;
    auto tiles_of = [&](int i) {
      return split(D[i].tiles, wg + 1, nwg) - split(D[i].tiles, wg, nwg);
    };
    auto complete = [&](int i) {
      return lds_load(&sh.tiles_done[i % kDmaXBufs]) >= tiles_of(i);
    };
    auto finish_one = [&](int i) {
      const DmaDesc& d = D[i];
      const int b = i % kDmaXBufs;
      const int r0 = split(d.tiles, wg, nwg) * d.tr;
      int r1 = split(d.tiles, wg + 1, nwg) * d.tr;
      if (r1 > d.N) r1 = d.N;
      const uint16_t* yb = ybuf + b * ybuf_rows;
      if (!d.signal) {
        Q4_GLOBAL uint16_t* Y = (Q4_GLOBAL uint16_t*)d.Y;
        for (int r = r0 + lane; r < r1; r += 64) Y[r] = yb[r - r0];
      } else {
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(d.Y, 0, 0x7FFFFFFF, 0x00020000);
        for (int r = r0 + lane; r < r1; r += 64)
          __builtin_amdgcn_raw_buffer_store_b16(yb[r - r0], ry, 2 * r, 0, kCoherent);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        if (lane == 0)
          __hip_atomic_fetch_add(&done[i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      wait_lds();
      if (lane == 0) lds_store(&sh.tiles_done[b], 0);   // buffer b is reused by i + NX
    };
    auto finish_upto = [&](int last, bool block) {
      while (next_fin <= last && next_fin < n) {
        if (!complete(next_fin)) {
          if (!block) return;
          for (unsigned it = 0; !complete(next_fin); ++it) {
            if (it > kSpinLimit) { err[0] = 1u; break; }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        finish_one(next_fin);
        next_fin += kSync;
      }
    };
    for (int k = me; k < n; k += kSync) {
      const DmaDesc& d = D[k];
      const int G = d.G, nblk = 4 * G;
      finish_upto(k - kSync, false);
      if (k >= kDmaXBufs) finish_upto(k - kDmaXBufs, true);
      const bool coherent = d.dep >= 0;
      if (coherent) {
        if (d.dep % kSync == me) finish_upto(d.dep, true);
        for (unsigned it = 0;
             __hip_atomic_load(&done[d.dep], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             (unsigned)nwg;
             ++it) {
          if (it > kSpinLimit) { err[0] = 2u; break; }
          finish_upto(k - kSync, false);
          __builtin_amdgcn_s_sleep(1);
        }
      }
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(d.X), 0, 0x7FFFFFFF, 0x00020000);
      const Q4_GLOBAL u32x4_g* X = (const Q4_GLOBAL u32x4_g*)d.X;
      const int b = k % kDmaXBufs;
      uint4* xb = xbuf + b * 4 * maxG;
      float* cb = cbuf + b * maxG;
      for (int i0 = 0; i0 < nblk; i0 += 8 * 64) {
        uint4 v[8];
        if (coherent) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 64 + lane;
            if (i < nblk) {
              const u32x4_g tv = __builtin_amdgcn_raw_buffer_load_b128(rx, 16 * i, 0, kCoherent);
              v[u] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * 64 + lane;
            if (i < nblk) {
              const u32x4_g tv = X[i];
              v[u] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 64 + lane;
          if (i0 + u * 64 < nblk) {
            float se = 0.f, so = 0.f;
            if (i < nblk) {
              xb[(i & 3) * maxG + (i >> 2)] = pair_order(v[u]);
              const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const h2_t h = bits<h2_t>(wv[e]);
                se += (float)h[0];
                so += (float)h[1];
              }
            }
            se += dpp<0xB1>(se);
            so += dpp<0xB1>(so);
            se += dpp<0x4E>(se);
            so += dpp<0x4E>(so);
            if (i < nblk && (i & 3) == 0) cb[i >> 2] = __builtin_fmaf(1031.0f, se, 71.0f * so);
          }
        }
      }
      wait_lds();
      if (lane == 0) lds_store(&sh.x_ready[b], k);
    }
    finish_upto(n - 1, true);
    if (me == 0) {
      for (unsigned it = 0; !complete(n - 1) && next_fin <= n - 1; ++it) {
        if (it > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(1);
      }
      // the last GEMV's owner has finished it once every tile is done; wait for
      // the whole tile count before reading the error word
      int total = 0;
      for (int i = 0; i < n; ++i) total += tiles_of(i);
      for (unsigned it = 0; lds_load(&sh.next_tile) < total + kCompute; ++it) {
        if (it > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) {
        const int e = lds_load(&sh.err);
        if (e) err[0] = (unsigned)e;
      }
    }
    return;
  }

  // ------------------------------------------------------------ compute waves
  const Nibbles nb = make_nibbles();
  const uint8_t* ring_b = reinterpret_cast<const uint8_t*>(ring);
  int total = 0;
  for (int i = 0; i < n; ++i) total += split(D[i].tiles, wg + 1, nwg) - split(D[i].tiles, wg, nwg);
  int cur_j = -1, lg = 2, lpr = 4, C = 1, G = 1, tr0 = 0, xi = 0;
  while (true) {
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(&sh.next_tile, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t >= total) break;
    const int slot = t % kSlots;
    for (unsigned it = 0; lds_load(&sh.slot_tile[slot]) != t; ++it) {
      if (it > kSpinLimit) { lds_store(&sh.err, 5); break; }
      __builtin_amdgcn_s_sleep(1);
    }
    const int j = __builtin_amdgcn_readfirstlane(lds_load(&sh.slot_j[slot]));
    const int row0 = __builtin_amdgcn_readfirstlane(lds_load(&sh.slot_row0[slot]));
    const int rows = __builtin_amdgcn_readfirstlane(lds_load(&sh.slot_rows[slot]));
    if (j != cur_j) {
      const DmaDesc& d = D[j];
      cur_j = j;
      lg = d.lpr_log2;
      lpr = 1 << lg;
      C = d.C;
      G = d.G;
      tr0 = split(d.tiles, wg, nwg) * d.tr;
      xi = j % kDmaXBufs;
    }
    for (unsigned it = 0; lds_load(&sh.x_ready[xi]) != j; ++it) {
      if (it > kSpinLimit) { lds_store(&sh.err, 3); break; }
      __builtin_amdgcn_s_sleep(1);
    }
    const int li = lane & (lpr - 1);
    const int rps = 64 >> lg;
    const int steps = (rows + rps - 1) / rps;
    const uint8_t* wl = ring_b + slot * kSlotBytes + ((lane >> lg) * G + li) * 16;
    const uint8_t* sl = ring_b + slot * kSlotBytes + kSlotWordBytes + ((lane >> lg) * G + li) * 2;
    const uint4* xb = xbuf + xi * 4 * maxG + li;
    const float* cb = cbuf + xi * maxG + li;
    const int step_w = rps * G * 16, step_s = rps * G * 2;   // bytes between row-steps
    for (int s = 0; s < steps; s += 2) {
      const bool two = s + 1 < steps;
      float acc0 = 0.f, acc1 = 0.f;
      for (int tg = 0; tg < C; ++tg) {
        uint4 x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * tg];
        const float nbias = -cb[lpr * tg];
        const int go = lpr * tg;
        const uint4 w0 = *reinterpret_cast<const uint4*>(wl + s * step_w + go * 16);
        const uint16_t s0 = *reinterpret_cast<const uint16_t*>(sl + s * step_s + go * 2);
        acc0 = __builtin_fmaf(group_dot(w0, x, nbias, nb), (float)bits<_Float16>(s0), acc0);
        if (two) {
          const uint4 w1 = *reinterpret_cast<const uint4*>(wl + (s + 1) * step_w + go * 16);
          const uint16_t s1 = *reinterpret_cast<const uint16_t*>(sl + (s + 1) * step_s + go * 2);
          acc1 = __builtin_fmaf(group_dot(w1, x, nbias, nb), (float)bits<_Float16>(s1), acc1);
        }
      }
      acc0 = team_sum(acc0, lg);
      acc1 = team_sum(acc1, lg);
      if (li == 0) {
        const int r = row0 + s * rps + (lane >> lg);
        if (r < row0 + rows) ybuf[xi * ybuf_rows + (r - tr0)] = bits<uint16_t>((_Float16)acc0);
        if (two && r + rps < row0 + rows)
          ybuf[xi * ybuf_rows + (r + rps - tr0)] = bits<uint16_t>((_Float16)acc1);
      }
    }
    wait_lds();
    if (lane == 0) {
      lds_store(&sh.slot_free[slot], t);
      __hip_atomic_fetch_add(&sh.tiles_done[xi], 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

__global__ void k_zero_dma(unsigned* __restrict__ p, int count) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

DmaPlan plan_step_dma(const DeviceInfo& dev, const StepLayer* layers, int64_t n,
                      const std::vector<int>& dep, const std::vector<int>& signal) {
  DmaPlan p;
  p.ok = false;
  if (n < 1) return p;
  p.grid = dev.cus;
  p.desc.resize((size_t)n);
  int maxG = 8, ybuf_rows = 8;
  for (int64_t k = 0; k < n; ++k) {
    const StepLayer& L = layers[k];
    if (L.K % 256 || L.K > 8192) return p;
    if (reinterpret_cast<uintptr_t>(L.scales) % 16) return p;
    const int G = (int)(L.K / 32);
    // lanes per row: a power of two dividing G with G / lanes <= 8 groups per
    // lane, preferring about 4 groups per lane
    int lg = 0;
    while ((1 << (lg + 1)) <= 64 && G % (1 << (lg + 1)) == 0 && (G >> lg) > 4) ++lg;
    const int lpr = 1 << lg, C = G / lpr;
    if (C > 8 || lpr * C != G) return p;
    const int rps = 64 / lpr;
    int tr = (kSlotWordBytes / (G * 16)) / rps * rps;       // rows per tile
    if (tr < rps) return p;
    DmaDesc& s = p.desc[(size_t)k];
    s.W = reinterpret_cast<const uint4*>(L.words);
    s.S = L.scales;
    s.X = reinterpret_cast<const uint4*>(L.x);
    s.Y = L.y;
    s.N = (int)L.N;
    s.G = G;
    s.lpr_log2 = lg;
    s.C = C;
    s.tr = tr;
    s.tiles = (int)((L.N + tr - 1) / tr);
    s.dep = dep[(size_t)k];
    s.signal = signal[(size_t)k];
    if (G > maxG) maxG = G;
    const int rows_wg = ((s.tiles + p.grid - 1) / p.grid) * tr;
    if (rows_wg > ybuf_rows) ybuf_rows = rows_wg;
  }
  p.maxG = maxG;
  p.ybuf_rows = (ybuf_rows + 7) & ~7;
  p.lds_bytes = (size_t)kSlots * kSlotBytes +
                (size_t)kDmaXBufs * ((size_t)4 * maxG * 16 + (size_t)maxG * 4 +
                                     (size_t)p.ybuf_rows * 2);
  p.counters = (int)n + 4;
  p.ok = p.lds_bytes + 512 <= dev.lds_per_block;
  return p;
}

size_t step_dma_workspace_bytes(const DmaPlan& p) {
  return ((size_t)p.counters * sizeof(unsigned) + 255) & ~(size_t)255;
}

hipError_t step_dma_occupancy(const DmaPlan& p, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, reinterpret_cast<const void*>(k_step_dma), kStepThreads, p.lds_bytes);
}

hipError_t launch_step_dma(const DmaPlan& p, const DmaDesc* dev_desc, void* ws, hipStream_t s) {
  unsigned* done = static_cast<unsigned*>(ws);
  unsigned* err = done + (p.counters - 1);
  hipLaunchKernelGGL(k_zero_dma, dim3(1), dim3(256), 0, s, done, p.counters);
  if (hipError_t e = hipGetLastError()) return e;
  if (p.lds_bytes > 65536) {
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_step_dma),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)p.lds_bytes))
      return e;
  }
  int n = (int)p.desc.size(), maxG = p.maxG, yr = p.ybuf_rows;
  void* args[] = {(void*)&dev_desc, (void*)&n, (void*)&done, (void*)&err, (void*)&maxG,
                  (void*)&yr};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_step_dma), dim3(p.grid),
                                    dim3(kStepThreads), args, (unsigned)p.lds_bytes, s);
}

}  // namespace q4
