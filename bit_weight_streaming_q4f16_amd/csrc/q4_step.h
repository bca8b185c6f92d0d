// Internal interface of the persistent decode-step kernel (q4_step.hip).
#pragma once

#include <vector>

#include "q4_internal.h"

namespace q4 {

constexpr int kStepThreads = 1024;   // one workgroup of 16 waves per compute unit

// The control block at the start of a decode-step workspace (uint32 words), read
// and written by the persistent kernels: the error word, the hand-over epoch, the
// exit count, then (from word kCtlWords) one completion counter per descriptor.
constexpr int kCtlErr = 0;     // a bounded wait ran out: code | (GEMV + 1) << 8 (0: none)
constexpr int kCtlEpoch = 1;   // epoch the last launch tagged its handed-over values with
constexpr int kCtlExit = 2;    // workgroups past their work in the current launch
constexpr int kCtlWords = 64;  // 256 bytes
// Error codes of kCtlErr (the wait that ran out).
constexpr unsigned kErrLocal = 1;    // sync wave: this workgroup's compute waves on a GEMV
constexpr unsigned kErrCounter = 2;  // sync wave: a GEMV's completion counter
constexpr unsigned kErrX = 3;        // compute wave: a GEMV's x in LDS
constexpr unsigned kErrTag = 4;      // sync wave: a GEMV's tagged hand-over
constexpr unsigned kErrRegion = 5;   // sync wave (small M): an LDS region's previous user

// Record the first bounded wait that ran out (any racing writer's value is valid).
__device__ __forceinline__ void report_error(unsigned* ctl, unsigned code, int gemv) {
  __hip_atomic_store(ctl + kCtlErr, code | ((unsigned)(gemv + 1) << 8), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kXBufs = 8;            // x buffers: waves may run up to 8 GEMVs apart

// Descriptor flags.
constexpr int kPublish = 1;  // later descriptors wait for this one's completion counter
constexpr int kTagOut = 2;   // y also goes to the workspace as epoch-tagged pairs
constexpr int kTagIn = 4;    // x is read from an earlier descriptor's tagged pairs
constexpr int kPairs = 8;    // workgroup shares are split in pairs of row-steps (even rows)
constexpr int kSiluMul = 16; // x is [gate | up]: the input is fp16(silu(gate) * up)
constexpr int kQ3 = 32;      // q3f16_1 words: 12 bytes per group (W is then a byte address)
constexpr int kAffine = 64;  // MLX affine: a scale and a bias per two groups (S, Bs [N][G/2]),
                             // weight = s * q + b; bf16 unless kAffineF16
constexpr int kAffineF16 = 128;

// One GEMV as the persistent kernel reads it (device-resident table, 80 bytes).
struct StepDesc {
  const uint4* W;        // words, one uint4 per 32-weight group: [N][G]
  const uint16_t* S;     // scales [N][G]
  const uint4* X;        // x as blocks of 8 halves: [4G]
  uint16_t* Y;           // y [N]
  int N, G;              // rows, groups per row (K / 32)
  int16_t lpr_log2;      // lanes per row = 2^lpr_log2 (4..64)
  int16_t C;             // groups per lane (<= 4)
  int steps;             // row-steps: ceil(N / (64 / lanes per row))
  int dep;               // descriptor that must be complete before x is read (-1: none)
  int flags;             // kPublish | kTagOut | kTagIn | kPairs | kSiluMul
  int sbase, srem;       // workgroup w owns row-steps from w * sbase + min(w, srem)
                         // (pairs of row-steps with kPairs): split evenly over the
                         // grid, the first srem get one more
  int tag_in;            // kTagIn: workspace byte offset of the tagged pairs x is read from
  int tag_out;           // kTagOut: workspace byte offset of this GEMV's tagged pairs
  const uint16_t* Bs;    // kAffine: biases [N][G/2] (NULL otherwise)
};
static_assert(sizeof(StepDesc) == 80, "StepDesc layout");

struct StepLayer {
  const uint32_t* words;
  const uint16_t* scales;
  const uint16_t* x;
  uint16_t* y;
  int64_t N, K;
  uint32_t x_op;          // Q4_X_PLAIN (x is [M][K]) or Q4_X_SILU_MUL (x is [M][2K])
  uint32_t format;        // 0: q4f16_1, or Q4_FMT_Q3F16_1, Q4_FMT_AF4_G64(_F16) (M = 1 only)
  const uint16_t* biases; // the affine formats' biases, NULL otherwise
  int64_t x_cols() const { return x_op ? 2 * K : K; }
};

struct StepPlan {
  bool ok = false;       // false: the list needs the one-kernel-per-GEMV path
  int grid = 0;          // workgroups (one per compute unit)
  int maxG = 0;
  int ybuf_rows = 0;
  size_t tag_base = 0;   // workspace byte offset of the tagged pairs (after the counters)
  size_t tag_bytes = 0;  // their size (0: no descriptor hands its y over that way)
  bool cross_wg = false; // some descriptor waits for others on every workgroup: all
                         // workgroups must be resident at once (cooperative launch)
  int nx = 0;            // x buffers (kXBufs, or 4 in range mode)
  // Range mode (no dependencies): per workgroup {first row-step, end row-step,
  // first GEMV, last GEMV} of the row-steps of all GEMVs laid end to end,
  // balanced by weight bytes.  Empty otherwise.
  std::vector<int> ranges;
  size_t lds_bytes = 0;
  bool affine = false;   // some descriptor is affine (kAffine)
  std::vector<StepDesc> desc;
};

// What launching a planned list needs, as plain data (kept in the caller's plan
// buffer).  Workspace layout: control block and completion counters, tagged
// pairs, then the device tables (descriptors, then the ranges if any).
struct StepLaunch {
  int32_t kind;          // 1: k_step (M = 1), 2: k_step_mfma (2 <= M <= 8)
  int32_t n, grid, M;
  int32_t nx, maxG, ybuf_rows, stage_off;
  int32_t cross_wg, has_ranges;
  uint32_t lds_bytes;
  uint32_t affine;       // k_step: the list holds affine GEMVs (the variant that loads biases)
  uint64_t table_off, ranges_off, table_bytes;
  uint64_t clear_bytes;  // bytes cleared at set-up: control block, counters, tags
  uint64_t ws_bytes;     // total workspace
};

// ordered: every descriptor waits for its predecessor (a chain of dependent GEMVs);
// otherwise only for earlier descriptors whose memory it shares.
StepPlan plan_step(const DeviceInfo& d, const StepLayer* layers, int64_t n, bool ordered,
                   bool tags = true);
// The launch record and the table bytes of a plan.
StepLaunch step_launch_of(const StepPlan& p);
void step_table_bytes(const StepPlan& p, std::vector<uint8_t>* out);
hipError_t step_occupancy(const StepPlan& p, int* blocks_per_cu);
// The kernel's attribute for the plan's LDS (once per process and device).
hipError_t step_prepare(const StepLaunch& L);
// Enqueue one launch of a planned list (tables and counters already in ws).
hipError_t launch_step(const StepLaunch& L, void* ws, hipStream_t s);

// Set-up helpers shared by both persistent kernels, kernels only (no copy from
// host memory, no allocation, capturable): write `bytes` (a multiple of 4) of
// host data to device memory through kernel arguments, and zero device words.
hipError_t write_table(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t zero_words(void* dst, size_t words, hipStream_t s);

}  // namespace q4
