// Host-side kernel launchers (internal).  Arguments are validated by the C-ABI layer before these
// are called; every size passed here is non-empty.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace fp8bq {

hipError_t launch_quant_1x128(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, uint8_t* q,
                              int64_t ldq, float* s, int64_t lds, hipStream_t st);
hipError_t launch_quant_128x1(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, uint8_t* qt,
                              int64_t ldqt, float* st_, int64_t ldst, hipStream_t st);
// Both activation layouts (1x128 row groups with format fr, 128x1 column groups with format fc,
// transposed) from one read of x; R % 128 == 0 and C % 128 == 0.
hipError_t launch_quant_dual(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fr, uint8_t* q,
                             int64_t ldq, float* s, int64_t lds, int fc, uint8_t* qt, int64_t ldqt, float* st_,
                             int64_t ldst, hipStream_t st);
// Weight codes and scales as launch_quant_128x128 plus the transposed codes qt [K, N].
hipError_t launch_quant_128x128_dual(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                                     int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt, hipStream_t st);
hipError_t launch_quant_128x128(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                                int64_t ldq, float* s, int64_t lds, hipStream_t st);

// Several weights quantized as launch_quant_128x128_dual in one launch (all of one input type and
// format).  Job j covers blocks start[j] .. start[j+1]-1 (nkb[j] = K_j / 128 tiles per tile row);
// only jobs with at least one tile are listed, so start is strictly increasing and start[count] is
// the grid size.  Passed to the kernel by value (about 1.2 KB of kernel arguments).
constexpr int kMaxWeightJobs = 16;
struct WeightDualBatch {
  const void* w[kMaxWeightJobs];
  uint8_t* q[kMaxWeightJobs];
  float* s[kMaxWeightJobs];
  uint8_t* qt[kMaxWeightJobs];
  int64_t ldw[kMaxWeightJobs], ldq[kMaxWeightJobs], lds[kMaxWeightJobs], ldqt[kMaxWeightJobs];
  uint32_t nkb[kMaxWeightJobs];
  uint32_t start[kMaxWeightJobs + 1];
  int count;
};
hipError_t launch_quant_weights_dual(const WeightDualBatch& b, int wt, int fmt, hipStream_t st);

// Per-tensor delayed scaling: the running amax *amax is updated with max|x| (beta = EMA decay) and
// gives the scale *s; q[R, C] gets the codes of x's BF16 copy, and qt[C, R] the same codes
// transposed when qt is non-null (then R % 128 == 0).  ws holds kTensorAmaxBlocks partial maxima
// and the running amax as it was (kTensorWorkspace bytes).
constexpr int kTensorAmaxBlocks = 1024;
constexpr size_t kTensorWorkspace = (kTensorAmaxBlocks + 64) * sizeof(float);
int tensor_amax_blocks(int64_t R);
// Device address of the library's own scratch for the delayed quantizer on device dev (the current
// device; looked up on its first use there, then cached).
hipError_t tensor_scratch(int dev, float** out);
hipError_t launch_quant_tensor_delayed(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, float* amax,
                                       double beta, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s,
                                       void* ws, hipStream_t st);

// Streaming copy of bytes (a multiple of 16; both pointers 16-byte aligned, ranges disjoint) with a
// grid sized from the device's compute-unit count: the bandwidth reference.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, int cus, hipStream_t st);

// One scaled FP8 GEMM in "TN" form: C[m, n] = sum_kb sa(kb, m) * sb(kb, n) * sum_{k in kb} A[m, k] B[n, k],
// where A [Mr, K] and B [Nc, K] are both contiguous along the contraction.
//   sa(kb, m) = sa[kb * ldsa + m * sa_mstride]
//   sb(kb, n) = sb[kb * sb_kstride + (n / 128) * sb_nstride]   (SbMode::kBlock128)
//   sb(kb, n) = sb[kb * sb_kstride + n]                         (SbMode::kColumn)
struct GemmDesc {
  const uint8_t* a;
  int64_t lda;
  const uint8_t* b;
  int64_t ldb;
  const float* sa;
  int64_t ldsa;
  int64_t sa_mstride;  // 1: one A scale per row; 0: one scale for all rows (per-tensor scaling)
  const float* sb;
  int64_t sb_kstride;
  int64_t sb_nstride;
  void* c;
  int64_t ldc;
  int64_t M, N, K;
  int fa, fb;    // FP8 format of A and B
  int out_f32;   // 0: BF16 output, 1: FP32 output, 2: FP32 output accumulated into (c += result)
  int sb_mode;   // SbMode
};

hipError_t launch_gemm(int op, const GemmDesc& d, const GemmPlan& plan, void* ws, hipStream_t st);

// Byte-matrix transpose: dst[c * ldd + r] = src[r * lds + c] for r < R, c < C (R, C multiples of 128).
hipError_t launch_transpose_u8(const uint8_t* src, int64_t lds, uint8_t* dst, int64_t ldd, int64_t R, int64_t C,
                               hipStream_t st);

// Fill n bytes of dst with zeros (used when a GEMM's contraction length is 0).
hipError_t launch_zero_fill(void* dst, int64_t rows, int64_t row_bytes, int64_t ld_bytes, hipStream_t st);

}  // namespace fp8bq
