// Internal interface of the whole-token persistent kernel (q4_tok.hip): one
// launch runs every stage of one or more decode steps of the decode loop.
#pragma once

#include "q4_internal.h"
#include "q4_step.h"

namespace q4 {

constexpr int kTokThreads = 1024;    // one workgroup of 16 waves per compute unit
constexpr int kTokBuffers = 4;       // LDS x buffers (stages in flight per workgroup)

// Control-block words used by the token kernel beside the error word, the epoch
// and the exit count of the step kernels (q4_step.h).
constexpr int kCtlKey = 8;           // uint64 (words 8, 9): argmax key of the step
constexpr int kCtlArrive = 10;       // workgroups that have added their key
constexpr int kCtlToken = 12;        // uint64 (words 12, 13): {token, epoch}
// Error words of the token kernel carry this bit beside the wait code
// (q4_step.h kErr*); the descriptor field is the stage within the step.
constexpr unsigned kErrTokenKernel = 0x80;

// Stage flags.
constexpr int kTokEmbed = 1;   // input: the token's embedding row, normalised (h = row)
constexpr int kTokNorm = 2;    // input: h = fp16(residual + tagged delta), normalised
constexpr int kTokGlu = 4;     // rows i and nout + i give silu_mul_h of the two results
constexpr int kTokArgmax = 8;  // outputs are the logits: also their argmax
// Neither kTokEmbed nor kTokNorm: the input is the previous stage's tagged output.

// One stage of a step as the kernel reads it (device-resident table, 80 bytes).
struct TokStage {
  const uint4* W;          // words [rows][G]
  const uint16_t* S;       // scales [rows][G]
  const uint16_t* gamma;   // normalised stages: the RMSNorm weight, fp16 [32 G]
  uint16_t* out;           // outputs [0, nplain) as plain fp16 (NULL if nplain == 0)
  int rows;                // matrix rows (2 nout with kTokGlu)
  int G;                   // groups per row (K / 32)
  int16_t lg, C;           // 2^lg lanes per row, C groups per lane (C 2^lg >= G)
  int nout;                // outputs
  int flags;               // kTok*
  int nplain;              // outputs [0, nplain) go to `out`, the rest are tagged
  int tag_in;              // workspace byte offset of the tagged input (x or delta)
  int tag_out;             // workspace byte offset of the tagged outputs [nplain, nout)
  int nburst;              // bursts: ceil(nout / outputs per burst)
  int sbase, srem;         // workgroup w owns bursts from w * sbase + min(w, srem)
  int pad;
};
static_assert(sizeof(TokStage) == 80, "TokStage layout");

// What a launch needs (kept in the caller's plan buffer).
struct TokLaunch {
  int32_t grid, stages, maxG, D;
  int32_t V, burst;
  uint32_t lds_bytes;
  float eps;
  uint64_t table_off;            // workspace offset of the stage table
  const uint32_t* embed_words;   // [V][D / 8]
  const uint16_t* embed_scales;  // [V][D / 32]
};

// Outputs per burst of a stage (bursts of `burst` items; an item is one row per
// team of 2^lg lanes).
inline int tok_outputs_per_burst(int burst, int lg, bool glu) {
  const int rows = burst * (64 >> lg);
  return glu ? rows / 2 : rows;
}

// LDS bytes of a launch: the x buffers (pair-ordered planes and offset terms),
// the residual, the per-wave output staging.
inline size_t tok_lds_bytes(int maxG, int D) {
  return (size_t)kTokBuffers * ((size_t)4 * maxG * 16 + (size_t)maxG * 4) + (size_t)2 * D +
         (size_t)12 * 64 * 4;
}

hipError_t tok_prepare(const TokLaunch& L);
// Enqueue one launch running `steps` decode steps: step t reads tokens[t] (t = 0
// from memory, later ones from the previous step's argmax) and writes
// tokens[t + 1]; logits: the last step's logits (NULL: the stage table's buffer).
hipError_t launch_tokens(const TokLaunch& L, void* ws, int32_t* tokens, int steps,
                         uint16_t* logits, hipStream_t s);

}  // namespace q4
