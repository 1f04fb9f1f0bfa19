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

// w [R, C] FP32 (in place), g [R, C] BF16 (gt = 0) or FP32 (gt = 1); C % 8 == 0.  norms: NULL or
// two floats (||g||, ||w|| after the update and before the projection).
hipError_t launch_hyperball_step(float* w, int64_t ldw, const void* g, int gt, int64_t ldg, int64_t R, int64_t C,
                                 double lr, double wd, double eps, double radius, float* norms, void* ws,
                                 hipStream_t st);

}  // namespace fp8bq
