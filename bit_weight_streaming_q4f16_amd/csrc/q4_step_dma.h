// Internal interface of the LDS-ring persistent decode-step kernel (q4_step_dma.hip).
#pragma once

#include <vector>

#include "q4_step.h"

namespace q4 {

constexpr int kLoaders = 4;                  // loader waves (one per SIMD)
constexpr int kSlots = 12;                   // LDS ring slots, kSlots / kLoaders per loader
constexpr int kSlotWordBytes = 8192;         // words of one tile (at most)
constexpr int kSlotScaleBytes = 1024;        // room for its scales (one 1 KB copy)
constexpr int kSlotBytes = kSlotWordBytes + kSlotScaleBytes;
constexpr int kDmaXBufs = 2;                 // x buffers

struct DmaDesc {
  const uint4* W;        // words [N][G] (one uint4 per group)
  const uint16_t* S;     // scales [N][G]
  const uint4* X;        // x [4G] blocks of 8 halves
  uint16_t* Y;           // y [N]
  int N, G;
  int lpr_log2, C;       // 2^lpr_log2 lanes per row, C groups per lane, exactly G
  int tr, tiles;         // rows per tile, tiles of the GEMV
  int dep, signal;       // as in StepDesc
};
static_assert(sizeof(DmaDesc) == 64, "DmaDesc layout");

struct DmaPlan {
  bool ok = false;
  int grid = 0, maxG = 0, ybuf_rows = 0, counters = 0;
  size_t lds_bytes = 0;
  std::vector<DmaDesc> desc;
};

// dep / signal: per descriptor, as computed for the register kernel.
DmaPlan plan_step_dma(const DeviceInfo& d, const StepLayer* layers, int64_t n,
                      const std::vector<int>& dep, const std::vector<int>& signal);
size_t step_dma_workspace_bytes(const DmaPlan& p);
hipError_t step_dma_occupancy(const DmaPlan& p, int* blocks_per_cu);
hipError_t launch_step_dma(const DmaPlan& p, const DmaDesc* dev_desc, void* ws, hipStream_t s);

}  // namespace q4
