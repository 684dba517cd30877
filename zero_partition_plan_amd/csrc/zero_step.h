// Internal declarations shared by the step's host entry points (zero_step.hip) and its kernel
// instantiations (zero_step_kernels.hip, compiled once per replica/output dtype pair so the many
// kernel variants build in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_shard.h"

#ifndef ZERO_ADAM_SUB
#define ZERO_ADAM_SUB 1            // 4-element groups per thread per tile in the Adam kernel
#endif
#ifndef ZERO_ADAM_BLOCK
#define ZERO_ADAM_BLOCK 64         // threads per block of the Adam kernel (one wave)
#endif
#ifndef ZERO_REP_BATCH
#define ZERO_REP_BATCH 8           // replica loads issued together before they are summed
#endif

namespace zero {
namespace step {

constexpr int kBlock = 256;                 // the squared-norm finish
constexpr int kAdamBlock = ZERO_ADAM_BLOCK;
constexpr uint64_t kAdamTile = (uint64_t)kAdamBlock * 4 * ZERO_ADAM_SUB;
constexpr uint64_t kRedTile = 256;          // reduce tile: one squared-norm partial each
constexpr uint64_t kMaxGrid = 1u << 24;     // blocks per launch; keeps grid * block below 2^32

struct RepPtrs {
  const void* p[ZERO_MAX_REPLICAS];
};

struct StepScalars {
  float gs;  // grad_scale
  float b1, b2, c1, c2, ss, bc, e, dec, w;
};

// Step inputs that live in device memory: the grad scale (zero_clip_scale writes it) and,
// optionally, the step t with a table of per-step constants (entry t-1). A t outside
// [1, table_len] makes every block exit without writing: the update is refused.
struct DevCtl {
  const float* gs;
  const zero_adam_scalars* table;  // NULL: the constants passed in StepScalars
  const int64_t* step;
  uint32_t table_len;
};

// Where the 16-bit arrays sit relative to 4-byte words. The vector path reads and writes whole
// 4-byte words; a 16-bit array that starts at an odd element (2 bytes past a word) is read from
// the word before it and realigned in registers, and a 16-bit output there is written as whole
// words assembled across neighbouring lanes, with 16-bit stores only at the ends of each wave's
// run. Both are 0 when every 16-bit array starts on a word.
struct Phase {
  uint64_t rep_odd;  // bit k: replica k starts at an odd element
  uint32_t out_odd;  // the 16-bit output starts at an odd element
};

struct AdamArgs {
  RepPtrs reps;
  int nrep;
  uint64_t ntiles;      // whole tiles, from element 0
  uint64_t n;
  StepScalars sc;
  float *P, *M, *V;
  void* out;
  const int32_t* skip;
  DevCtl dc;            // dc.gs == NULL: everything from sc
  hipStream_t stream;
  bool fused_tail;      // the shard ends in a partial tile: the last grid's extra block takes it
  Phase ph;
};

struct ReduceArgs {
  RepPtrs reps;
  int nrep;
  uint64_t n;
  float* G;
  int32_t* flag;
  double* partials;
  double sq_scale;
  hipStream_t stream;
  Phase ph;
};

inline uint64_t red_tiles(uint64_t n) { return n / kRedTile + (n % kRedTile != 0); }  // no wrap

// Enqueue the fused update for replica dtype RDT and output dtype ODT (ZERO_F32: no output).
template <int RDT, int ODT>
void launch_adam(const AdamArgs& a, bool l2);

// Enqueue the reduce pass for replica dtype RDT.
template <int RDT>
void launch_reduce(const ReduceArgs& a);

}  // namespace step
}  // namespace zero
