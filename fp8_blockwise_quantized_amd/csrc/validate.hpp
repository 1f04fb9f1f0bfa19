// Argument validation for the C-ABI entry points (pure host C++, no HIP calls), so every error path
// can be exercised on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fp8bq {

// Status codes mirror fp8bq_status in include/fp8bq.h.
enum Status : int {
  kOk = 0,
  kErrNull = 1,
  kErrShape = 2,
  kErrLd = 3,
  kErrAlign = 4,
  kErrDtype = 5,
  kErrFormat = 6,
  kErrWorkspace = 7,
  kErrDevice = 8,
  kErrLaunch = 9,
  kErrOverlap = 10,
  kErrValue = 11,
};

// A row-major matrix view for validation: base pointer, rows, columns, leading dimension (elements),
// element size (bytes).
struct Mat {
  const void* p;
  int64_t rows, cols, ld;
  int esize;
};

// Checks pointer non-null, 16-byte alignment, ld >= cols and ld*esize % 16 == 0 (if align_ld).
int check_mat(const Mat& m, bool align_ld);
// Byte ranges of two non-empty matrices intersect.
bool overlaps(const Mat& a, const Mat& b);

int validate_quant_1x128(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* q,
                         int64_t ldq, const void* s, int64_t lds, bool* empty);
int validate_quant_128x1(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* qt,
                         int64_t ldqt, const void* st, int64_t ldst, bool* empty);
int validate_quant_dual(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fr, const void* q, int64_t ldq,
                        const void* s, int64_t lds, int fc, const void* qt, int64_t ldqt, const void* st,
                        int64_t ldst, bool* empty);
int validate_quant_128x128_dual(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, const void* q,
                                int64_t ldq, const void* s, int64_t lds, const void* qt, int64_t ldqt, bool* empty);
int validate_quant_128x128(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, const void* q,
                           int64_t ldq, const void* s, int64_t lds, bool* empty);
// Several weights: count in [0, max_jobs]; each job as validate_quant_128x128_dual (empty[j] set per
// job); no job's outputs may overlap another job's input or outputs.  Job fields are passed as
// parallel arrays so this stays free of the public header's types.
struct WeightJobArgs {
  const void* w; int64_t N, K, ldw;
  const void* q; int64_t ldq;
  const void* s; int64_t lds;
  const void* qt; int64_t ldqt;
};
int validate_quant_weights_dual(const WeightJobArgs* jobs, int count, int max_jobs, int wt, int fmt, bool* empty);

// Per-tensor delayed scaling: x [R, C] (C % 128 == 0), running amax and scale one float each (4-byte
// aligned), q [R, C], optional qt [C, R] (then R % 128 == 0), beta in [0, 1], ws >= ws_needed bytes.
// ws_needed == 0 validates a call that takes no workspace (ws and ws_bytes are then ignored).
int validate_quant_tensor(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, const void* amax,
                          double beta, const void* q, int64_t ldq, const void* qt, int64_t ldqt, const void* s,
                          const void* ws, size_t ws_bytes, size_t ws_needed, bool* empty);

// Hyperball step: w [R, C] FP32, g [R, C] (BF16 or FP32), C % 8 == 0; lr >= 0, wd >= 0, eps > 0,
// radius >= 0, all finite; norms NULL or two 4-byte-aligned floats; ws >= ws_needed bytes.
int validate_hyperball(const void* w, int64_t ldw, const void* g, int gt, int64_t ldg, int64_t R, int64_t C,
                       double lr, double wd, double eps, double radius, const void* norms, const void* ws,
                       size_t ws_bytes, size_t ws_needed, bool* empty);

// Streaming copy: src and dst non-null and 16-byte aligned, bytes a multiple of 16 below 2^48, the two
// ranges disjoint.
int validate_stream_copy(const void* src, const void* dst, size_t bytes, bool* empty);

// Several Hyperball steps: count in [0, max_jobs]; each job as validate_hyperball (empty[j] set per
// job; lr, wd, eps shared); no job's written memory (w, norms) may overlap another job's w, g or
// norms, or the workspace.  ws >= ws_needed bytes when any job is non-empty.
struct HyperballJobArgs {
  const void* w; int64_t ldw;
  const void* g; int64_t ldg;
  int64_t R, C;
  double radius;
  const void* norms;
};
int validate_hyperball_batch(const HyperballJobArgs* jobs, int count, int max_jobs, int gt, double lr, double wd,
                             double eps, const void* ws, size_t ws_bytes, size_t ws_needed, bool* empty);

// The three GEMMs share one validator: op selects the operand shapes.
struct GemmArgs {
  int op;
  int64_t M, N, K;
  const void* qa; int64_t ldqa; const void* sa; int64_t ldsa; int fa;
  const void* qb; int64_t ldqb; const void* sb; int64_t ldsb; int fb;
  const void* out; int out_t; int64_t ldout;
  const void* ws; size_t ws_bytes;
};
// *empty: the output has no elements.  *zero_fill: the output is non-empty but the contraction is
// empty, so the result is all zeros.  ws_needed: bytes the plan needs.
int validate_gemm(const GemmArgs& g, size_t ws_needed, bool* empty, bool* zero_fill);

}  // namespace fp8bq
