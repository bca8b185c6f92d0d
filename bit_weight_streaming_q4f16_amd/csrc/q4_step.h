// Internal interface of the persistent decode-step kernel (q4_step.hip).
#pragma once

#include <vector>

#include "q4_internal.h"

namespace q4 {

constexpr int kStepThreads = 1024;   // one workgroup of 16 waves per compute unit
constexpr int kXBufs = 8;            // x buffers: waves may run up to 8 GEMVs apart

// Descriptor flags.
constexpr int kPublish = 1;  // later descriptors wait for this one's completion counter
constexpr int kTagOut = 2;   // y also goes to the workspace as epoch-tagged pairs
constexpr int kTagIn = 4;    // x is read from an earlier descriptor's tagged pairs
constexpr int kPairs = 8;    // workgroup shares are split in pairs of row-steps (even rows)
constexpr int kSiluMul = 16; // x is [gate | up]: the input is fp16(silu(gate) * up)

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
  int pad[2];
};
static_assert(sizeof(StepDesc) == 80, "StepDesc layout");

struct StepLayer {
  const uint32_t* words;
  const uint16_t* scales;
  const uint16_t* x;
  uint16_t* y;
  int64_t N, K;
  uint32_t x_op;          // Q4_X_PLAIN (x is [M][K]) or Q4_X_SILU_MUL (x is [M][2K])
  int64_t x_cols() const { return x_op ? 2 * K : K; }
};

struct StepPlan {
  bool ok = false;       // false: the list needs the one-kernel-per-GEMV path
  int grid = 0;          // workgroups (one per compute unit)
  int maxG = 0;
  int ybuf_rows = 0;
  int counters = 0;      // completion counters, exit counter, spare, error word
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
  std::vector<StepDesc> desc;
};

// ordered: every descriptor waits for its predecessor (a chain of dependent GEMVs);
// otherwise only for earlier descriptors whose memory it shares.
StepPlan plan_step(const DeviceInfo& d, const StepLayer* layers, int64_t n, bool ordered,
                   bool tags = true);
size_t step_workspace_bytes(const StepPlan& p);
// dev_desc: p.desc copied to device memory.  Zeroes the counters in ws (unless
// ws_clean: they are already zero, as the kernel leaves them), then runs the
// cooperative kernel.
// dev_ranges: p.ranges copied to device memory (nullptr when p.ranges is empty).
hipError_t launch_step(const StepPlan& p, const StepDesc* dev_desc, const int4* dev_ranges,
                       void* ws, bool ws_clean, hipStream_t s);
// The epoch the next launch tags its handed-over pairs with (never 0, increasing).
uint32_t next_step_epoch();
hipError_t step_occupancy(const StepPlan& p, int* blocks_per_cu);

}  // namespace q4
