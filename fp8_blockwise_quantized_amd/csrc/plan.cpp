// Tile / launch planner (pure host C++).
#include "plan.hpp"

#include <cstdlib>

namespace fp8bq {

// FP8BQ_GEMM_TILE=<0..4> forces a tile shape (a TileShape value; tuning aid); read once.
static int forced_shape() {
  static const int v = [] {
    const char* e = std::getenv("FP8BQ_GEMM_TILE");
    const int x = e ? std::atoi(e) : -1;
    return (x >= 0 && x <= 4) ? x : -1;
  }();
  return v;
}

static int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }  // a >= 0, b > 0

// Time of one contraction block for one round of resident work units, in microseconds, measured
// on MI355X: two 128x128 workgroups per CU take ~1.2 us per block, one 256x256 workgroup ~2.05 us
// (4x the work for 1.7x the time: half the operand traffic per flop), four 64x64 workgroups ~0.94 us
// (half the work of two 128x128 ones for 0.8 of the time: that tile pays off only where the larger
// ones leave compute units idle, i.e. few output rows).
static double block_us(int shape) { return shape == k256x256 ? 2.05 : shape == k64x64 ? 0.94 : 1.2; }

// Cost model in microseconds: rounds of resident units x blocks per unit x block time, plus, for a
// split, a pass that writes and re-reads split x rows x cols FP32 partials and writes the output
// (~5 TB/s effective) and costs a fixed ~6 us as a launch of its own (measured: a 512-token fprop
// split in two took 18.9 us where 1024 tokens unsplit took 15.8).  Splitting pays off only when
// the tiles alone leave workgroup slots idle.
// A last round that fills only a fraction f of the slots runs faster than a full one (less
// contention for memory and power): it is charged (1 + f) / 2 of a round, as measured on MI355X
// (a half-full last round of 256x256 tiles took ~0.74 of a full one).
static double split_cost(int64_t rows, int64_t cols, int64_t nkb, int64_t slots, int shape, int s) {
  const int64_t tiles = cdiv(rows, tile_rows(shape)) * cdiv(cols, tile_cols(shape));
  const int64_t units = tiles * s;
  const int64_t full = units / slots;
  const double frac = (double)(units - full * slots) / (double)slots;
  const double rounds = (double)full + (frac > 0.0 ? 0.5 * (1.0 + frac) : 0.0);
  const double gemm_us = rounds * ((double)nkb / s) * block_us(shape);
  const double red_us = s > 1 ? 6.0 + (8.0 * s + 4.0) * (double)rows * (double)cols / 5.0e6 : 0.0;
  return gemm_us + red_us;
}

static int best_split(int64_t rows, int64_t cols, int64_t nkb, int64_t slots, int shape, double* cost) {
  int best = 1;
  double best_us = 0.0;
  for (int s = 1; s <= kMaxSplit; ++s) {
    if (s > 1 && nkb / s < 4) break;  // keep at least 4 blocks per unit
    const double us = split_cost(rows, cols, nkb, slots, shape, s);
    if (s == 1 || us < best_us * 0.97) {
      best = s;
      best_us = us;
    }
  }
  if (cost) *cost = best_us;
  return best;
}

GemmPlan plan_gemm(int op, int64_t M, int64_t N, int64_t K, int cu_count) {
  GemmPlan p;
  // Output shape and contraction length in the kernel's TN frame.
  int64_t rows, cols, contraction;
  if (op == kOpFprop || op == kOpTensor) {
    rows = M; cols = N; contraction = K;
  } else if (op == kOpDgrad || op == kOpDgradWt) {
    rows = M; cols = K; contraction = N;
  } else {
    rows = N; cols = K; contraction = M;
  }
  const int64_t cus = cu_count > 0 ? cu_count : 256;
  const int64_t nkb = contraction / 128;
  // one launch addresses its work units with 32 bits: at most 2^31 - 1 units of any tile shape and
  // split; sizes beyond that (far past any device memory) get an empty plan that the caller refuses
  const int64_t kMaxTiles128 = ((int64_t)1 << 28) - 1;
  const int64_t t128m = rows > 0 ? cdiv(rows, 128) : 0, t128n = cols > 0 ? cdiv(cols, 128) : 0;
  if (t128m > kMaxTiles128 || t128n > kMaxTiles128 || (t128n > 0 && t128m > kMaxTiles128 / t128n) ||
      nkb > ((int64_t)1 << 31) - 1 ||
      (op == kOpDgrad && (double)N * (double)K >= 4.611686018427388e18)) {
    p.fits = false;
    return p;
  }
  const bool work = rows > 0 && cols > 0 && nkb > 0;
  if (forced_shape() >= 0) {
    p.shape = forced_shape();
  } else if (work) {
    // the fastest tile shape under the cost model (ties go to the larger tile)
    double c64 = 0.0, c128 = 0.0, c256 = 0.0;
    best_split(rows, cols, nkb, cus * blocks_per_cu(k64x64), k64x64, &c64);
    best_split(rows, cols, nkb, cus * blocks_per_cu(k128x128), k128x128, &c128);
    best_split(rows, cols, nkb, cus * blocks_per_cu(k256x256), k256x256, &c256);
    p.shape = c256 <= c128 ? k256x256 : k128x128;
    if (c64 < (p.shape == k256x256 ? c256 : c128)) p.shape = k64x64;
  } else {
    p.shape = k128x128;
  }
  p.tile_m = tile_rows(p.shape);
  p.tile_n = tile_cols(p.shape);
  const int64_t slots = cus * blocks_per_cu(p.shape);
  p.tiles_m = cdiv(rows, p.tile_m);
  p.tiles_n = cdiv(cols, p.tile_n);
  p.split_k = work ? best_split(rows, cols, nkb, slots, p.shape, nullptr) : 1;
  // (a split is only chosen for few tiles; this keeps the unit count in 31 bits whatever the tile)
  if (p.split_k > 1 && p.tiles_m * p.tiles_n > (((int64_t)1 << 31) - 1) / p.split_k) p.split_k = 1;
  p.units = p.tiles_m * p.tiles_n * p.split_k;
  // persistent grid: one workgroup per slot (a multiple of 8, so each workgroup stays on one XCD's
  // range of tiles), or one per unit when there are fewer units
  int64_t g = slots >= 8 ? slots - slots % 8 : slots;  // (a device with fewer than 8 CUs: all of them)
  p.grid = p.units < g ? p.units : g;
  p.ws_gemm = p.split_k > 1 ? (size_t)p.split_k * (size_t)rows * (size_t)cols * 4 : 0;
  p.ws_transpose = (op == kOpDgrad) ? (size_t)N * (size_t)K : 0;
  // round the transpose buffer up so the partial sums that follow it stay 256-byte aligned
  p.ws_transpose = (p.ws_transpose + 255) & ~(size_t)255;
  return p;
}

}  // namespace fp8bq
