// Tile / launch planner (pure host C++).
#include "plan.hpp"

#include <cstdlib>

namespace fp8bq {

// FP8BQ_GEMM_VARIANT=<n> forces a tile variant (tuning aid); read once.
static int forced_variant() {
  static const int v = [] {
    const char* e = std::getenv("FP8BQ_GEMM_VARIANT");
    return e ? std::atoi(e) : -1;
  }();
  return v;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

GemmPlan plan_gemm(int op, int64_t M, int64_t N, int64_t K, int cu_count) {
  (void)cu_count;
  GemmPlan p;
  // Output shape and contraction length in the kernel's TN frame.
  int64_t rows, cols;
  if (op == kOpFprop) {
    rows = M; cols = N;
  } else if (op == kOpDgrad) {
    rows = M; cols = K;
  } else {
    rows = N; cols = K;
  }
  p.variant = kVar128x128;
  if (forced_variant() >= 0) p.variant = forced_variant();
  p.tile_m = p.variant == kVar256x256 ? 256 : 128;
  p.tile_n = p.variant == kVar256x256 ? 256 : 128;
  p.split_k = 1;
  p.tiles_m = cdiv(rows, p.tile_m);
  p.tiles_n = cdiv(cols, p.tile_n);
  p.grid = p.tiles_m * p.tiles_n * p.split_k;
  p.ws_gemm = 0;
  p.ws_transpose = (op == kOpDgrad) ? (size_t)N * (size_t)K : 0;
  // round the transpose buffer up so the split-K area that may follow it stays 256-byte aligned
  p.ws_transpose = (p.ws_transpose + 255) & ~(size_t)255;
  return p;
}

}  // namespace fp8bq
