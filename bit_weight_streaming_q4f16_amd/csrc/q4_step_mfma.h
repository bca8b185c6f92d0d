// Internal interface of the persistent small-M decode-step kernel (q4_step_mfma.hip).
#pragma once

#include <vector>

#include "q4_step.h"

namespace q4 {

// One GEMV as the small-M kernel reads it (device-resident table, 64 bytes).
struct MStepDesc {
  const uint4* W;        // words [N][G] (one uint4 per group)
  const uint16_t* S;     // scales [N][G]
  const uint4* X;        // X [M][K] as blocks of 8 halves
  uint16_t* Y;           // Y [M][N]
  int N, G;
  int tbase, trem;       // 16-row tiles split over the grid: workgroup w owns tiles from
                         // w * tbase + min(w, trem), the first trem get one more; or,
                         // with trem < 0 (range mode), tbase is the GEMV's first tile
                         // among the tiles of all GEMVs laid end to end
  int dep, signal;       // as in StepDesc
  int xoff;              // byte offset of the GEMV's LDS region (X, y rows)
  int rel;               // GEMV whose LDS region overlaps this one (-1: none): it must
                         // be finished before this one's X is staged
};
static_assert(sizeof(MStepDesc) == 64, "MStepDesc layout");

struct MStepPlan {
  bool ok = false;
  bool cross_wg = false;     // some descriptor waits for another on every workgroup
  int grid = 0, M = 0;
  size_t lds_bytes = 0;
  int stage_off = 0;         // LDS offset of the compute waves' load stages
  std::vector<MStepDesc> desc;
  // range mode (no dependencies): per workgroup {first tile, end tile, first GEMV,
  // last GEMV} of the tiles of all GEMVs laid end to end; empty otherwise
  std::vector<int> ranges;
};

// Persistent kernel for 2 <= M <= 8: every K a multiple of 128 and at most 8192,
// every GEMV's LDS region (16 K + 2 M rows bytes) within the LDS.
MStepPlan plan_step_mfma(const DeviceInfo& d, const StepLayer* layers, int64_t n, int M,
                         bool ordered);
// Launch record (workspace: control block and counters, then the tables) and
// table bytes of a plan.
StepLaunch step_mfma_launch_of(const MStepPlan& p);
void step_mfma_table_bytes(const MStepPlan& p, std::vector<uint8_t>* out);
hipError_t step_mfma_occupancy(const MStepPlan& p, int* blocks_per_cu);
hipError_t step_mfma_prepare(const StepLaunch& L);
hipError_t launch_step_mfma(const StepLaunch& L, void* ws, hipStream_t s);

}  // namespace q4
