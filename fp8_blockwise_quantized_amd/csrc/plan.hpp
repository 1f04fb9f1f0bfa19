// Tile / launch planner for the scaled FP8 GEMMs (pure host C++, no HIP calls).
//
// Given the product (fprop, dgrad, wgrad), its sizes and the device's compute-unit count, picks the
// split of the contraction across workgroups, the persistent grid, and the workspace it needs.
// Deterministic for equal inputs.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fp8bq {

enum SbMode : int { kSbBlock128 = 0, kSbColumn = 1 };
// kOpDgradWt: dgrad on weight codes already transposed (W^T [K, N]): the dgrad kernel, no transpose.
// kOpTensor: Y[M, N] = sa sb A[M, K] B[N, K]^T with one scale per operand (per-tensor scaling): the
// fprop kernel with broadcast scales, planned as fprop.
enum Op : int { kOpFprop = 0, kOpDgrad = 1, kOpWgrad = 2, kOpDgradWt = 3, kOpTensor = 4 };

// Workgroup tile shapes (output rows x columns of one work unit):
//   k128x128: 4 waves of 64x64, two workgroups per CU;
//   k128x256 / k256x128: 8 waves of 64x64, one workgroup per CU (tuning shapes, never planned);
//   k256x256: 8 waves of 128x64, one workgroup per CU;
//   k64x64: 4 waves of 16x64, four workgroups per CU (few output rows: 4x the tiles of 128x128).
enum TileShape : int { k128x128 = 0, k128x256 = 1, k256x128 = 2, k256x256 = 3, k64x64 = 4 };
inline int tile_rows(int shape) {
  return shape == k64x64 ? 64 : (shape == k256x128 || shape == k256x256) ? 256 : 128;
}
inline int tile_cols(int shape) {
  return shape == k64x64 ? 64 : (shape == k128x256 || shape == k256x256) ? 256 : 128;
}
inline int blocks_per_cu(int shape) { return shape == k64x64 ? 4 : shape == k128x128 ? 2 : 1; }
constexpr int kMaxSplit = 8;

struct GemmPlan {
  int shape = k128x128;
  int tile_m = 128;
  int tile_n = 128;
  int split_k = 1;    // contraction split across work units (FP32 partials reduced afterwards)
  int64_t tiles_m = 0, tiles_n = 0;
  int64_t units = 0;  // tiles x split
  int64_t grid = 0;   // persistent workgroups launched
  size_t ws_gemm = 0;       // workspace for split partial sums
  size_t ws_transpose = 0;  // workspace for dgrad's transposed weight codes
  // false when the product is too large for one launch (more than 2^28 - 1 output tiles of
  // 128x128, or a dgrad transpose buffer past 2^62 bytes); the plan is then empty
  bool fits = true;
  size_t ws_total() const { return ws_transpose + ws_gemm; }
};

// M, N, K follow the C-ABI meaning for each op (fprop: Y[M,N] = X[M,K] W[N,K]^T; dgrad: dX[M,K] =
// dY[M,N] W[N,K]; wgrad: dW[N,K] = dY[M,N]^T X[M,K]).
GemmPlan plan_gemm(int op, int64_t M, int64_t N, int64_t K, int cu_count);

}  // namespace fp8bq
