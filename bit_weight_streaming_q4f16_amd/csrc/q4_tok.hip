// Whole-token persistent kernel: every stage of one or more decode steps of the
// decode loop (Zero TVM documentation, "Decode loop": per block the qkv
// projection, attention, o, the residual add with RMSNorm, gate/up, SiLU-multiply,
// down, the residual add with RMSNorm; then the LM head and the greedy argmax)
// in ONE launch.  The pages' host-side lever is to submit a whole token in one
// command (everything-webgpu AI.md, "Multi-step decoding"); here a whole token,
// or several, is one kernel, so the weight stream of the next projection is in
// flight while the current one finishes, and no projection pays a kernel
// boundary.  The norms are folded into the projection they feed, as
// Q4_MODEL_FACTORED_NORM does with separate kernels: the projection stages
// h * gamma and scales its fp32 results by 1 / rms(h).  Attention runs at a
// single position (its output is the value part of qkv).
//
// One workgroup of 16 waves per compute unit (cooperative launch: all resident):
//  * 12 compute waves.  A workgroup owns an even share of the bursts of every
//    stage (a burst: two items, an item one row per team of 2^lg lanes, each
//    lane holding up to 4 groups).  The workgroup's bursts of all stages, in
//    order, are dealt round-robin to its compute waves, and each wave keeps two
//    bursts in flight: the loads of its next burst are issued before it waits
//    for the input of the current one, so the weights of the next stage stream
//    while the current stage waits for its input.  A wave writes its outputs
//    itself: fp16 pairs tagged with the step's epoch (one 64-bit store, written
//    through to the coherence point) for the stage that reads them, plain
//    stores for the q/k rows and the logits.  The stores are issued after the
//    next burst's loads, so no wait for a burst's loads also waits for a store.
//  * 4 sync waves.  Each owns a quarter of the input groups of every stage: it
//    polls the producing stage's tagged pairs until all carry this step's
//    epoch, forms the input (normalised stages: h = fp16(residual + delta),
//    kept as the workgroup's own copy of the residual stream in LDS, and
//    fp16(h * gamma) with the partial sum of h^2), stages it pair-ordered in one
//    of four LDS buffers with the per-group offset terms, and counts itself in.
//    Sync wave 0 also ends a step: once every compute wave is past the logits
//    it adds the workgroup's argmax key to the step's key, and the last
//    workgroup to do so publishes the token (tagged with the epoch) for the
//    next step's embedding row.
// Every residual copy is updated from the same tagged values in the same way,
// so all workgroups hold the same residual stream without exchanging it.
// Every wait is bounded; running out sets the error word (stage within the
// step, with kErrTokenKernel) and the kernel still finishes.
#include <algorithm>
#include <cstring>

#include "q4_tok.h"
#include "q4_device.h"

namespace q4 {
namespace {

constexpr int kWaves = kTokThreads / 64;     // 16
constexpr int kSync = 4;
constexpr int kCompute = kWaves - kSync;     // 12
constexpr int NX = kTokBuffers;
constexpr unsigned kSpin = 1u << 24;         // LDS waits (about a second)
constexpr unsigned kTagSpin = 1u << 18;      // polls of tagged pairs (a memory round trip each)

struct Shared {
  int x_cnt[NX];             // sync-wave stagings completed per buffer (monotonic)
  int done[NX];              // compute waves past the buffer's stage (monotonic)
  float ssp[NX][kSync];      // normalised stages: each sync wave's sum of h^2
  unsigned long long key;    // the workgroup's argmax key of the current step
  int err;                   // a compute wave's wait ran out: stage + 1
};

__device__ __forceinline__ int wg_first(int sbase, int srem, int wg) {
  return wg * sbase + (wg < srem ? wg : srem);
}

// The hand-over epoch of step t of this launch: one past the last launch's, then
// one more per step, never 0 (tags start zeroed).
__device__ __forceinline__ unsigned epoch_of(unsigned base, int t) {
  return 1u + (unsigned)(((unsigned long long)base + (unsigned)t) % 0xFFFFFFFFull);
}

// The fields of a stage a compute wave needs, read with scalar loads issued as
// inline assembly: as ordinary loads they become vector loads (the compiler
// cannot prove the table unchanged across the kernel's own stores), and using
// one would first drain the weight loads in flight.
struct StageRegs {
  const Q4_GLOBAL uint4* W;
  const Q4_GLOBAL uint16_t* S;
  uint16_t* out;
  int rows, G, lg, C, nout, flags, nplain, tag_out, sbase, srem;
};
__device__ __forceinline__ StageRegs read_stage(const TokStage* d) {
  u32x8_s a, b;
  u32x4_g c;
  asm volatile(
      "s_load_dwordx8 %0, %3, 0x0\n\t"
      "s_load_dwordx8 %1, %3, 0x20\n\t"
      "s_load_dwordx4 %2, %3, 0x40\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(a), "=&s"(b), "=&s"(c)
      : "s"(d));
  static_assert(offsetof(TokStage, S) == 8 && offsetof(TokStage, out) == 24 &&
                    offsetof(TokStage, rows) == 32 && offsetof(TokStage, lg) == 40 &&
                    offsetof(TokStage, nout) == 44 && offsetof(TokStage, flags) == 48 &&
                    offsetof(TokStage, nplain) == 52 && offsetof(TokStage, tag_out) == 60 &&
                    offsetof(TokStage, nburst) == 64 && offsetof(TokStage, sbase) == 68 &&
                    offsetof(TokStage, srem) == 72,
                "stage offsets read by the compute waves");
  StageRegs r;
  r.W = (const Q4_GLOBAL uint4*)(((uint64_t)a[1] << 32) | a[0]);
  r.S = (const Q4_GLOBAL uint16_t*)(((uint64_t)a[3] << 32) | a[2]);
  r.out = (uint16_t*)(((uint64_t)a[7] << 32) | a[6]);
  r.rows = (int)b[0];
  r.G = (int)b[1];
  r.lg = (int)(b[2] & 0xFFFFu);
  r.C = (int)(b[2] >> 16);
  r.nout = (int)b[3];
  r.flags = (int)b[4];
  r.nplain = (int)b[5];
  r.tag_out = (int)b[7];
  r.sbase = (int)c[1];
  r.srem = (int)c[2];
  return r;
}

// Argmax key of an output: its order as an fp16 value (NaN skipped, -0 taken as
// +0) above the complement of its index (ties go to the lowest index); 0: none.
__device__ __forceinline__ unsigned long long argmax_key(uint32_t h, int j, bool ok) {
  if (!ok || (h & 0x7FFFu) > 0x7C00u) return 0ull;
  if (h == 0x8000u) h = 0u;
  const uint32_t ord = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
  return ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)j);
}

// LDS layout (dynamic): xbuf [NX][4][maxG] pair-ordered planes (uint4), cbuf
// [NX][maxG] offset terms, res [D / 8] blocks of the residual, wout [12][64]
// team results of each compute wave's current burst.
template <int B>
__global__ __launch_bounds__(kTokThreads) void k_tokens(
    const TokStage* __restrict__ T, int S, int steps, unsigned* __restrict__ ctl, int maxG, int D,
    float eps, const uint32_t* __restrict__ EW, const uint16_t* __restrict__ ES, int V,
    int32_t* __restrict__ tokens, uint16_t* __restrict__ logits) {
  extern __shared__ uint4 smem[];
  __shared__ Shared sh;
  uint4* const xbuf = smem;
  float* const cbuf = reinterpret_cast<float*>(smem + NX * 4 * maxG);
  uint4* const res = reinterpret_cast<uint4*>(cbuf + NX * maxG);
  float* const wout = reinterpret_cast<float*>(res + D / 8);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x, nwg = gridDim.x;
  const unsigned base = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (threadIdx.x < NX) {
    sh.x_cnt[threadIdx.x] = 0;
    sh.done[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    sh.key = 0ull;
    sh.err = 0;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rws =
      __builtin_amdgcn_make_buffer_rsrc(ctl, 0, 0x7FFFFFFF, kRsrcFlags);

  if (wave < kSync) {
    // ------------------------------------------------------------- sync waves
    const int me = wave;
    const Nibbles nbs = make_nibbles();
    const uint4 w7 = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
    int tok = 0;
    for (int t = 0; t < steps; ++t) {
      const unsigned e = epoch_of(base, t);
      for (int sl = 0; sl < S; ++sl) {
        const int s = t * S + sl, b = s % NX, u = s / NX;
        const TokStage& d = T[sl];
        const int G = d.G, flags = d.flags, tag_in = d.tag_in;
        const bool normed = (flags & (kTokEmbed | kTokNorm)) != 0;
        const int g0 = me * G / kSync, g1 = (me + 1) * G / kSync, nbm = 4 * (g1 - g0);
        uint4* const xb = xbuf + b * 4 * maxG;
        float* const cb = cbuf + b * maxG;
        // the buffer's previous stage is behind every compute wave
        for (unsigned it = 0; u > 0 && lds_load(&sh.done[b]) < kCompute * u; ++it) {
          if (it > kSpin / 8) { report_error(ctl, kErrLocal | kErrTokenKernel, sl); break; }
          __builtin_amdgcn_s_sleep(8);
        }
        uint4 gm[4], v[4];
        if (normed) {
          const uint4* gamma = reinterpret_cast<const uint4*>(d.gamma);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int j = lane + 64 * k;
            gm[k] = j < nbm ? gamma[4 * g0 + j] : make_uint4(0u, 0u, 0u, 0u);
          }
        }
        if (flags & kTokEmbed) {
          if (t == 0) {
            tok = tokens[0];
          } else {
            // the previous step's token, published by its last workgroup
            const unsigned ep = epoch_of(base, t - 1);
            unsigned long long w = 0ull;
            for (unsigned it = 0;; ++it) {
              w = __hip_atomic_load(reinterpret_cast<unsigned long long*>(ctl + kCtlToken),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if ((unsigned)(w >> 32) == ep) break;
              if (it > kTagSpin) { report_error(ctl, kErrTag | kErrTokenKernel, sl); break; }
              __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            tok = (int)(unsigned)w;
          }
          tok = __builtin_amdgcn_readfirstlane(tok);
          const bool ok = tok >= 0 && tok < V;
          // the embedding row: fp16((q - 7) * s) per weight; NaN for a token
          // outside the vocabulary
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int j = lane + 64 * k;
            v[k] = make_uint4(0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u);
            if (j < nbm && ok) {
              const int i = 4 * g0 + j;
              const uint32_t w = EW[(int64_t)tok * (D / 8) + i];
              const float sc = half_to_float(ES[(int64_t)tok * G + (i >> 2)]);
              h8_t h;
#pragma unroll
              for (int q = 0; q < 8; ++q)
                h[q] = (_Float16)((float)((int)((w >> (4 * q)) & 0xFu) - 7) * sc);
              v[k] = bits<uint4>(h);
            }
          }
        } else {
          // block i = tagged pairs 4i .. 4i + 3 of the producing stage: taken once
          // all four carry this step's epoch, re-read until then
          unsigned pend = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[k] = make_uint4(0u, 0u, 0u, 0u);
            if (lane + 64 * k < nbm) pend |= 1u << k;
          }
          for (unsigned it = 0;; ++it) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              if (pend & (1u << k)) {
                const int i = 4 * g0 + lane + 64 * k;
                const u32x4_g a = __builtin_amdgcn_raw_buffer_load_b128(rws, tag_in + 32 * i, 0,
                                                                        kCoherent);
                const u32x4_g c2 = __builtin_amdgcn_raw_buffer_load_b128(
                    rws, tag_in + 32 * i + 16, 0, kCoherent);
                if (a[1] == e && a[3] == e && c2[1] == e && c2[3] == e) {
                  v[k] = make_uint4(a[0], a[2], c2[0], c2[2]);
                  pend &= ~(1u << k);
                }
              }
            }
            if (!__builtin_amdgcn_ballot_w64(pend != 0u)) break;
            if (it > kTagSpin) { report_error(ctl, kErrTag | kErrTokenKernel, sl); break; }
            __builtin_amdgcn_s_sleep(1);
          }
          if (flags & kTokNorm) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int j = lane + 64 * k;
              if (j < nbm)   // h = fp16(residual + delta): one native fp16 add
                v[k] = bits<uint4>(bits<h8_t>(res[4 * g0 + j]) + bits<h8_t>(v[k]));
            }
          }
        }
        // stage: normalised stages keep h as the residual and stage fp16(h * gamma)
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int j = lane + 64 * k;
          if (j < nbm) {
            const int i = 4 * g0 + j;
            uint4 x = v[k];
            if (normed) {
              res[i] = v[k];
              const h8_t h = bits<h8_t>(v[k]), g8 = bits<h8_t>(gm[k]);
              h8_t o;
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const float f = (float)h[q];
                ss = __builtin_fmaf(f, f, ss);
                o[q] = (_Float16)(f * (float)g8[q]);
              }
              x = bits<uint4>(o);
            }
            xb[(i & 3) * maxG + (i >> 2)] = pair_order(x);
          }
        }
        wait_lds();
        // per group the offset term: the compute waves' chain over codes all 7
        // with this x (see nibble_group_dot), read back from the planes
        for (int g = g0 + lane; g < g1; g += 64) {
          uint4 xq[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) xq[q] = xb[q * maxG + g];
          cb[g] = nibble_group_dot(w7, xq, nbs);
        }
        if (me == kSync - 1) {
          // groups past G up to the padded count read x = 0 and offset 0
          const int Gp = (1 << d.lg) * d.C;
          for (int i = 4 * G + lane; i < 4 * Gp; i += 64) {
            xb[(i & 3) * maxG + (i >> 2)] = make_uint4(0u, 0u, 0u, 0u);
            if ((i & 3) == 0) cb[i >> 2] = 0.f;
          }
        }
        if (normed) {
          ss = team_sum_lg(ss, 6);
          if (lane == 0) sh.ssp[b][me] = ss;
        }
        wait_lds();
        if (lane == 0)
          __hip_atomic_fetch_add(&sh.x_cnt[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((flags & kTokArgmax) && me == 0) {
          // every compute wave is past the logits: add this workgroup's key; the
          // last workgroup reads the step's key, resets it and the count, and
          // publishes the token
          for (unsigned it = 0; lds_load(&sh.done[b]) < kCompute * (u + 1); ++it) {
            if (it > kSpin / 8) { report_error(ctl, kErrLocal | kErrTokenKernel, sl); break; }
            __builtin_amdgcn_s_sleep(8);
          }
          if (lane == 0) {
            unsigned long long* const gkey = reinterpret_cast<unsigned long long*>(ctl + kCtlKey);
            const unsigned long long k = __hip_atomic_exchange(
                &sh.key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (k) __hip_atomic_fetch_max(gkey, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned old = __hip_atomic_fetch_add(ctl + kCtlArrive, 1u, __ATOMIC_ACQ_REL,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            if (old == (unsigned)nwg - 1u) {
              const unsigned long long kk =
                  __hip_atomic_load(gkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              const int next = kk ? (int)(0xFFFFFFFFu - (uint32_t)kk) : 0;
              tokens[t + 1] = next;
              __hip_atomic_store(gkey, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(ctl + kCtlArrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(reinterpret_cast<unsigned long long*>(ctl + kCtlToken),
                                 (unsigned long long)(uint32_t)next | ((unsigned long long)e << 32),
                                 __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
  } else {
    // ---------------------------------------------------------- compute waves
    const int c = wave - kSync;
    const Nibbles nb = make_nibbles();
    const int total = steps * S;
    float* const wo = wout + c * 64;
    // Cursor over this workgroup's bursts of all stages of all steps, in order;
    // this wave takes positions c, c + 12, ...: stage cs (of the launch), stage
    // csl of the step, position cr among the workgroup's cnt bursts of it.
    int cs = 0, csl = 0, cr = c, ccnt = 0, cbb0 = 0;
    StageRegs R{};
    int vo[4] = {0, 0, 0, 0};
    auto load = [&](int sl) {
      R = read_stage(T + sl);
      const int lo = wg_first(R.sbase, R.srem, wg), hi = wg_first(R.sbase, R.srem, wg + 1);
      cbb0 = lo;
      ccnt = hi - lo;
      const int lpr = 1 << R.lg, tm = lane >> R.lg, li = lane & (lpr - 1);
      // a team's row relative to the item's first output: rows i (gate) and
      // nout + i (up) for the glue, row i otherwise
      const int roff = (R.flags & kTokGlu) ? (tm >> 1) + (tm & 1) * R.nout : tm;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool in = t < R.C && li + (t << R.lg) < R.G;
        // a slot past the row's groups reads past the resource: zeros, no access
        vo[t] = in ? (roff * R.G + li + (t << R.lg)) * 16 : 0x7FFFFFF0;
      }
    };
    auto settle = [&]() {
      while (cs < total && cr >= ccnt) {
        cr -= ccnt;
        ++cs;
        csl = csl + 1 == S ? 0 : csl + 1;
        if (cs < total) load(csl);
      }
    };
    if (total > 0) load(0);
    settle();

    struct Burst {
      uint4 w[B][4];
      uint16_t sc[B][4];
      int s, o;              // stage of the launch (total: none), first output
      StageRegs R;
    };
    // Every issue is the same 8 loads per item (4 dwordx4 of words, 4 ushort
    // scales); past the last burst the resources are empty, so no memory is read
    // and the wait counts stay exact.
    auto issue = [&](Burst& U) {
      const bool live = cs < total;
      const int rpi = 64 >> R.lg;
      const int opi = (R.flags & kTokGlu) ? rpi / 2 : rpi;
      const int o = live ? (cbb0 + cr) * B * opi : 0;
      U.s = live ? cs : total;
      U.o = o;
      U.R = R;
#pragma unroll
      for (int p = 0; p < B; ++p) {
        const int op = o + p * opi;
        const int64_t left = live && op < R.rows ? (int64_t)(R.rows - op) * R.G : 0;
        const uint32_t nw = left * 16 < 0xFFFFFFF0ll ? (uint32_t)(left * 16) : 0xFFFFFFF0u;
        const uint32_t ns = left * 2 < 0xFFFFFFF0ll ? (uint32_t)(left * 2) : 0xFFFFFFF0u;
        const __amdgpu_buffer_rsrc_t bw = __builtin_amdgcn_make_buffer_rsrc(
            live ? const_cast<uint4*>((const uint4*)(R.W + (int64_t)op * R.G)) : (uint4*)ctl, 0,
            (int)nw, kRsrcFlags);
        const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
            live ? const_cast<uint16_t*>((const uint16_t*)(R.S + (int64_t)op * R.G))
                 : (uint16_t*)ctl,
            0, (int)ns, kRsrcFlags);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4_g v = __builtin_amdgcn_raw_buffer_load_b128(bw, vo[t], 0, kNonTemporal);
          U.w[p][t] = make_uint4(v[0], v[1], v[2], v[3]);
          U.sc[p][t] = __builtin_amdgcn_raw_buffer_load_b16(bs, vo[t] >> 3, 0, 0);
        }
      }
    };
    auto next_pos = [&]() {
      cr += kCompute;
      settle();
    };

    int cur = 0;                     // stages [0, cur) signalled by this wave
    auto wait_x = [&](int s) {
      const int b = s % NX, need = kSync * (s / NX + 1);
      for (unsigned it = 0; lds_load(&sh.x_cnt[b]) < need; ++it) {
        if (it > kSpin) {
          __hip_atomic_store(&sh.err, s % S + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    };
    // signal the stages [cur, s): each once its x is staged (so the buffer's
    // counts stay in use order) and this wave's reads of it are done
    auto signal_upto = [&](int s) {
      for (; cur < s; ++cur) {
        wait_x(cur);
        wait_lds();
        if (lane == 0)
          __hip_atomic_fetch_add(&sh.done[cur % NX], 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };
    auto consume = [&](Burst& U) {
      const StageRegs& Q = U.R;
      signal_upto(U.s);
      wait_x(U.s);
      const int b = U.s % NX, lg = Q.lg, lpr = 1 << lg, li = lane & (lpr - 1),
                tm = lane >> lg, rpi = 64 >> lg;
      const bool glu = (Q.flags & kTokGlu) != 0;
      const uint4* xb = xbuf + b * 4 * maxG + li;
      const float* cb = cbuf + b * maxG + li;
      float rs = 1.f;
      if (Q.flags & (kTokEmbed | kTokNorm)) {
        const float tot = ((sh.ssp[b][0] + sh.ssp[b][1]) + sh.ssp[b][2]) + sh.ssp[b][3];
        rs = 1.f / __builtin_sqrtf(tot / (float)(32 * Q.G) + eps);
      }
      if (Q.C * lpr > Q.G) {             // padded rows: slots past G hold no weights
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool ok = li + lpr * t < Q.G;
#pragma unroll
          for (int p = 0; p < B; ++p) U.sc[p][t] = ok ? U.sc[p][t] : (uint16_t)0;
        }
      }
      float acc[B];
#pragma unroll
      for (int p = 0; p < B; ++p) acc[p] = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < Q.C) {
          uint4 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = xb[q * maxG + lpr * t];
          const float off = cb[lpr * t];
#pragma unroll
          for (int p = 0; p < B; ++p) {
            const float pd = nibble_group_dot(U.w[p][t], x, nb) - off;
            acc[p] = __builtin_fmaf(pd, (float)bits<_Float16>(U.sc[p][t]), acc[p]);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < B; ++p) {
        const float r = team_sum_lg(acc[p], lg) * kDotUnit * rs;
        if (li == 0) wo[p * rpi + tm] = r;
      }
      wait_lds();
      // lane m < opb / 2 writes outputs o + 2m and o + 2m + 1
      const int opb = glu ? B * rpi / 2 : B * rpi;
      const int m = lane < opb / 2 ? lane : opb / 2 - 1;
      const int j0 = U.o + 2 * m;
      const bool v0 = lane < opb / 2 && j0 < Q.nout, v1 = v0 && j0 + 1 < Q.nout;
      _Float16 lo, hi;
      if (glu) {
        lo = silu_mul_h((_Float16)wo[4 * m], (_Float16)wo[4 * m + 1]);
        hi = silu_mul_h((_Float16)wo[4 * m + 2], (_Float16)wo[4 * m + 3]);
      } else {
        lo = (_Float16)wo[2 * m];
        hi = (_Float16)wo[2 * m + 1];
      }
      const uint32_t lo16 = bits<uint16_t>(lo), hi16 = v1 ? (uint32_t)bits<uint16_t>(hi) : 0u;
      // A burst's outputs are all plain or all tagged.  Both kinds of store are
      // always issued (out-of-range offsets drop them), so every burst issues the
      // same three stores.
      const bool plain = U.o < Q.nplain;
      uint16_t* outp = (Q.flags & kTokArgmax) && logits ? logits : Q.out;
      const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
          outp ? outp : (uint16_t*)ctl, 0, outp ? 2 * Q.nplain : 0, kRsrcFlags);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)lo16, rp, plain && v0 ? 2 * j0 : 0x7FFFFFF0,
                                            0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hi16, rp,
                                            plain && v1 ? 2 * j0 + 2 : 0x7FFFFFF0, 0, 0);
      const int ntag = Q.nout - Q.nplain;
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<unsigned char*>(ctl) + Q.tag_out, 0, 4 * (ntag + (ntag & 1)),
          kRsrcFlags);
      const u32x2_g tv = {lo16 | (hi16 << 16), epoch_of(base, U.s / S)};
      __builtin_amdgcn_raw_buffer_store_b64(tv, rt, !plain && v0 ? 4 * (j0 - Q.nplain) : 0x7FFFFFF0,
                                            0, kCoherent);
      if (Q.flags & kTokArgmax) {
        const unsigned long long k0 = argmax_key(lo16, j0, v0), k1 = argmax_key(hi16, j0 + 1, v1);
        const unsigned long long k = k0 > k1 ? k0 : k1;
        if (k) __hip_atomic_fetch_max(&sh.key, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };

    // Two bursts in flight: the next one's loads go out before this one's wait
    // for its input.
    Burst A, Bq;
    issue(A);
    next_pos();
    while (A.s < total) {
      issue(Bq);
      next_pos();
      consume(A);
      if (Bq.s >= total) break;
      issue(A);
      next_pos();
      consume(Bq);
    }
    signal_upto(total);
  }

  // Hand the epoch to the next launch: the last workgroup to get here stores the
  // last step's (every workgroup read the old one when it started).
  __syncthreads();
  if (wave == 0 && lane == 0) {
    const int e = sh.err;
    if (e) report_error(ctl, kErrX | kErrTokenKernel, e - 1);
    const unsigned old =
        __hip_atomic_fetch_add(ctl + kCtlExit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (unsigned)nwg - 1u) {
      __hip_atomic_store(ctl + kCtlExit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctl + kCtlEpoch, epoch_of(base, steps - 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

constexpr int kTokBurst = 2;

}  // namespace

hipError_t tok_prepare(const TokLaunch& L) {
  if (L.lds_bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k_tokens<kTokBurst>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds_bytes);
}

hipError_t launch_tokens(const TokLaunch& L, void* ws, int32_t* tokens, int steps,
                         uint16_t* logits, hipStream_t s) {
  if (L.burst != kTokBurst) return hipErrorInvalidValue;
  const TokStage* T =
      reinterpret_cast<const TokStage*>(static_cast<uint8_t*>(ws) + L.table_off);
  unsigned* ctl = static_cast<unsigned*>(ws);
  int S = L.stages, maxG = L.maxG, D = L.D, V = L.V;
  float eps = L.eps;
  const uint32_t* EW = L.embed_words;
  const uint16_t* ES = L.embed_scales;
  void* args[] = {(void*)&T,   (void*)&S,  (void*)&steps, (void*)&ctl,    (void*)&maxG,
                  (void*)&D,   (void*)&eps, (void*)&EW,   (void*)&ES,     (void*)&V,
                  (void*)&tokens, (void*)&logits};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_tokens<kTokBurst>),
                                    dim3(L.grid), dim3(kTokThreads), args, L.lds_bytes, s);
}

}  // namespace q4
