// Tile / launch planner for the scaled FP8 GEMMs (pure host C++, no HIP calls).
//
// Given the product (fprop, dgrad, wgrad), its sizes and the device's compute-unit count, picks the
// workgroup tile, the split of the contraction across workgroups, the workspace it needs, and the
// grid.  Deterministic for equal inputs.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fp8bq {

enum SbMode : int { kSbBlock128 = 0, kSbColumn = 1 };
// Kernel tile variants: workgroup tile (rows x columns of the output) and wave layout.
enum Variant : int {
  kVar128x128 = 0,  // 4 waves (2x2) of 64x64, two workgroups per CU
  kVar256x256 = 1,  // 8 waves (2x4) of 128x64, one workgroup per CU
};
enum Op : int { kOpFprop = 0, kOpDgrad = 1, kOpWgrad = 2 };

struct GemmPlan {
  int tile_m = 128;   // output rows per workgroup
  int tile_n = 128;   // output columns per workgroup
  int variant = 0;    // kernel instance (tile shape / wave layout)
  int split_k = 1;    // contraction split across workgroups (partials reduced in the workspace)
  int64_t tiles_m = 0, tiles_n = 0;
  int64_t grid = 0;   // workgroups launched
  size_t ws_gemm = 0;       // workspace for split-K partial sums
  size_t ws_transpose = 0;  // workspace for dgrad's transposed weight codes
  size_t ws_total() const { return ws_transpose + ws_gemm; }
};

// M, N, K follow the C-ABI meaning for each op (fprop: Y[M,N] = X[M,K] W[N,K]^T; dgrad: dX[M,K] =
// dY[M,N] W[N,K]; wgrad: dW[N,K] = dY[M,N]^T X[M,K]).
GemmPlan plan_gemm(int op, int64_t M, int64_t N, int64_t K, int cu_count);

}  // namespace fp8bq
