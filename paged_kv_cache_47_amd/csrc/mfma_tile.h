// Row tile of the MFMA attention path, shared by the kernel and the plan.
#pragma once

#include "pa_internal.h"

namespace pa {

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 8
#endif
constexpr int kMfmaWaves = PA_PF_WAVES;          // waves per MFMA workgroup, 32 query rows each
constexpr int kMfmaRows = 32 * kMfmaWaves;
#ifndef PA_PF_BN
#define PA_PF_BN 64
#endif
constexpr int kMfmaBN = PA_PF_BN;   // keys per step of a row tile

// The keys row tile r of a sequence (L keys, Q query rows, group g) steps
// over: from the step-aligned start of its first row's window (0 without a
// window) to its last row's position, in 64-key steps.
struct TileSpan {
  int k0, kmax, steps;
};
__host__ __device__ __forceinline__ TileSpan tile_span(int L, int Q, int g, int r, int window) {
  const int rows = Q * g;
  const int last_row = (rows < (r + 1) * kMfmaRows ? rows : (r + 1) * kMfmaRows) - 1;
  const int kl = L - Q + last_row / g + 1;
  TileSpan t;
  t.kmax = L < kl ? L : kl;
  t.k0 = window_lo(L - Q + r * kMfmaRows / g, window) & ~(kMfmaBN - 1);
  t.steps = (t.kmax - t.k0 + kMfmaBN - 1) / kMfmaBN;
  return t;
}

// Split-K of long row tiles: a tile spanning more than `split` steps is cut
// into ceil(steps / split) parts of equal step counts (the last may be
// shorter; none is empty), each its own workgroup; their partial results are
// merged in log-sum-exp form.  split <= 0: never.
__host__ __device__ __forceinline__ int tile_parts(int steps, int split) {
  return split > 0 && steps > split ? (steps + split - 1) / split : 1;
}
__host__ __device__ __forceinline__ int part_steps(int steps, int parts) { return (steps + parts - 1) / parts; }

}  // namespace pa
