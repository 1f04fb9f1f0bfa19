// Hyperball weight update (internal launcher; arguments validated by the C-ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bq {

constexpr int kHyperballBlocks = 1024;  // most blocks of the sweeps (fp64 partials of each)
// workspace: per-block fp64 partial sums of g*g, w*w and w*g
constexpr size_t kHyperballWorkspace = 3 * kHyperballBlocks * sizeof(double);

int hyperball_blocks(int64_t R);

// Several matrices in one launch pair (all with gradients of one element type): job j is w[j] [R[j],
// C[j]] with gradient g[j], radius[j] (0: no projection) and norms[j] (NULL or two floats), its
// blocks start[j] .. start[j+1]-1 (hyperball_blocks(R[j]) of them; only non-empty jobs are listed),
// its partial sums at partial + j * 3 * kHyperballBlocks.  Passed by value (about 2.3 KB of kernel
// arguments).
constexpr int kMaxHyperballJobs = 32;
struct HyperballBatch {
  float* w[kMaxHyperballJobs];
  const void* g[kMaxHyperballJobs];
  int64_t ldw[kMaxHyperballJobs], ldg[kMaxHyperballJobs], R[kMaxHyperballJobs], C[kMaxHyperballJobs];
  double radius[kMaxHyperballJobs];
  float* norms[kMaxHyperballJobs];
  uint32_t start[kMaxHyperballJobs + 1];
  int count;
  double* partial;
};
hipError_t launch_hyperball_batch(const HyperballBatch& b, int gt, double lr, double wd, double eps, hipStream_t st);

// w [R, C] FP32 (in place), g [R, C] BF16 (gt = 0) or FP32 (gt = 1); C % 8 == 0.  norms: NULL or
// two floats (||g||, ||w|| after the update and before the projection).
hipError_t launch_hyperball_step(float* w, int64_t ldw, const void* g, int gt, int64_t ldg, int64_t R, int64_t C,
                                 double lr, double wd, double eps, double radius, float* norms, void* ws,
                                 hipStream_t st);

}  // namespace fp8bq
