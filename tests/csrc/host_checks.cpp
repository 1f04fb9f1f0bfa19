// Host-side checks of the argument validation and the GEMM planner (pure C++, no HIP), built with
// g++ and the address and undefined-behaviour sanitizers: random and extreme arguments (negative,
// zero and huge sizes, leading dimensions near 2^63, null and overlapping fake pointers) must never
// trigger undefined behaviour, every status must be a documented one, and every plan for a
// non-empty product must be consistent (split in 1..8, 1 <= grid <= units, workspace matching the
// split).  Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <random>

#include "plan.hpp"
#include "validate.hpp"

using namespace fp8bq;

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      if (failures < 20) std::fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static std::mt19937_64 rng(12345);

// sizes: mostly ordinary multiples of 128 and small ragged values, sometimes extreme
static int64_t pick_size() {
  switch (rng() % 8) {
    case 0: return -(int64_t)(rng() % 1000);
    case 1: return 0;
    case 2: return (int64_t)(rng() % 300);
    case 3: return 128 * (int64_t)(1 + rng() % 128);
    case 4: return 128 * (int64_t)(1 + rng() % 100000);
    case 5: return (int64_t)1 << (20 + rng() % 43);
    case 6: return INT64_MAX - (int64_t)(rng() % 1000);
    default: return 128 * (int64_t)(1 + rng() % 16);
  }
}
static int64_t pick_ld(int64_t cols) {
  switch (rng() % 5) {
    case 0: return cols;
    case 1: return cols > INT64_MAX - 200 ? cols : cols + 16 * (int64_t)(rng() % 8);
    case 2: return (int64_t)(rng() % 1000) - 10;
    case 3: return (int64_t)1 << (rng() % 63);
    default: return cols > 0 ? cols : 16;
  }
}
static const void* pick_ptr() {
  switch (rng() % 6) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<const void*>((uintptr_t)(rng() % (1ull << 47)) | 1);  // misaligned
    case 2: return reinterpret_cast<const void*>((uintptr_t)0x100000);                     // shared base
    default: return reinterpret_cast<const void*>((uintptr_t)((rng() % (1ull << 44)) & ~(uint64_t)15));
  }
}
static bool documented(int st) { return st >= kOk && st <= kErrValue; }

int main() {
  bool empty = false, zero = false;
  for (int it = 0; it < 200000; ++it) {
    const int64_t R = pick_size(), C = pick_size();
    const int xt = (int)(rng() % 3), fmt = (int)(rng() % 3);
    EXPECT(documented(validate_quant_1x128(pick_ptr(), xt, R, C, pick_ld(C), fmt, pick_ptr(), pick_ld(C), pick_ptr(),
                                           pick_ld(R), &empty)));
    EXPECT(documented(validate_quant_128x1(pick_ptr(), xt, R, C, pick_ld(C), fmt, pick_ptr(), pick_ld(R), pick_ptr(),
                                           pick_ld(C), &empty)));
    EXPECT(documented(validate_quant_dual(pick_ptr(), xt, R, C, pick_ld(C), fmt, pick_ptr(), pick_ld(C), pick_ptr(),
                                          pick_ld(R), fmt, pick_ptr(), pick_ld(R), pick_ptr(), pick_ld(C), &empty)));
    EXPECT(documented(validate_quant_128x128_dual(pick_ptr(), xt, R, C, pick_ld(C), fmt, pick_ptr(), pick_ld(C),
                                                  pick_ptr(), pick_ld(C / 128), pick_ptr(), pick_ld(R), &empty)));
    EXPECT(documented(validate_quant_tensor(pick_ptr(), xt, R, C, pick_ld(C), fmt, pick_ptr(), 0.5, pick_ptr(),
                                            pick_ld(C), rng() % 2 ? pick_ptr() : nullptr, pick_ld(R), pick_ptr(),
                                            pick_ptr(), (size_t)(rng() % 10000), 4352, &empty)));
    EXPECT(documented(validate_hyperball(pick_ptr(), pick_ld(C), pick_ptr(), xt, pick_ld(C), R, C, 1e-3, 0.1, 1e-8,
                                         (double)(rng() % 3), rng() % 2 ? pick_ptr() : nullptr, pick_ptr(),
                                         (size_t)(rng() % 100000), 16384, &empty)));
    WeightJobArgs jobs[3];
    bool je[3];
    for (auto& j : jobs)
      j = WeightJobArgs{pick_ptr(), R, C, pick_ld(C), pick_ptr(), pick_ld(C), pick_ptr(), pick_ld(C / 128),
                        pick_ptr(), pick_ld(R)};
    EXPECT(documented(validate_quant_weights_dual(jobs, (int)(rng() % 5) - 1, 16, xt, fmt, je)));
    HyperballJobArgs hjobs[3];
    bool he[3];
    for (auto& j : hjobs)
      j = HyperballJobArgs{pick_ptr(), pick_ld(C), pick_ptr(), pick_ld(C), rng() % 2 ? R : pick_size(), C,
                           (double)(rng() % 3) - 0.5, rng() % 2 ? pick_ptr() : nullptr};
    EXPECT(documented(validate_hyperball_batch(rng() % 8 ? hjobs : nullptr, (int)(rng() % 5) - 1, 32, xt, 1e-3, 0.1,
                                               1e-8, pick_ptr(), (size_t)(rng() % 200000), 3 * 24576, he)));
    EXPECT(documented(validate_stream_copy(pick_ptr(), pick_ptr(), (size_t)pick_size() * (rng() % 2 ? 16 : 1), &empty)));

    // the planner for any sizes, then the GEMM validator with its workspace requirement
    const int op = (int)(rng() % 5);
    const int64_t M = pick_size(), N = pick_size(), K = pick_size();
    const int cus = (int)(rng() % 4 == 0 ? rng() % 400 : 256);
    const GemmPlan p = plan_gemm(op, M, N, K, cus);
    EXPECT(p.split_k >= 1 && p.split_k <= kMaxSplit);
    EXPECT(p.units <= ((int64_t)1 << 31) - 1);  // the kernels count work units in 32 bits
    EXPECT(p.tile_m == tile_rows(p.shape) && p.tile_n == tile_cols(p.shape));
    if (p.units > 0) {
      EXPECT(p.grid >= 1 && p.grid <= p.units);
      EXPECT((p.split_k > 1) == (p.ws_gemm > 0));
    }
    GemmArgs g{op, M, N, K, pick_ptr(), pick_ld(K), pick_ptr(), pick_ld(M), fmt, pick_ptr(), pick_ld(K),
               pick_ptr(), pick_ld(K / 128), fmt, pick_ptr(), (int)(rng() % 4), pick_ld(N), pick_ptr(),
               (size_t)(rng() % (1u << 30))};
    EXPECT(documented(validate_gemm(g, p.ws_total(), &empty, &zero)));
  }
  // ordinary decoder shapes: the plans the bench relies on are well formed
  const int64_t shapes[][3] = {{16384, 2560, 2048}, {16384, 2048, 2048}, {16384, 11264, 2048}, {16384, 2048, 5632}};
  for (const auto& s : shapes)
    for (int op = 0; op < 5; ++op) {
      const GemmPlan p = plan_gemm(op, s[0], s[1], s[2], 256);
      EXPECT(p.units >= 1 && p.grid >= 1 && p.grid <= p.units && p.grid <= 512);
      EXPECT(p.tile_m == 128 || p.tile_m == 256);
    }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
