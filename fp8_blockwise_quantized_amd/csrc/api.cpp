// C-ABI entry points declared in include/fp8bq.h: validate, plan, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/fp8bq.h"
#include "launch.hpp"
#include "optim.hpp"
#include "plan.hpp"
#include "validate.hpp"

namespace fp8bq {

constexpr int kMaxDevices = 64;
// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other architecture.  Benign races (all writers
// store the same value).
static std::atomic<int> g_dev_state[kMaxDevices];
static std::atomic<int> g_dev_cus[kMaxDevices];

// Returns kOk if the current device is a gfx950; fills *cus with its compute-unit count and *index
// with its index (each if not null).
static int current_device(int* cus, int* index = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kErrDevice;
  }
  int state = g_dev_state[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return kErrDevice;
    }
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(state, std::memory_order_relaxed);
  }
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (index) *index = dev;
  return state == 1 ? kOk : kErrDevice;
}

static int cu_count_or_default() {
  int cus = 0;
  if (current_device(&cus) == kOk && cus > 0) return cus;
  return 256;
}

static int launched(hipError_t e) { return e == hipSuccess ? kOk : kErrLaunch; }

static int run_gemm(const GemmArgs& g, void* stream) {
  const int cus = cu_count_or_default();
  const GemmPlan plan = plan_gemm(g.op, g.M, g.N, g.K, cus);
  bool empty = false, zero = false;
  int st = validate_gemm(g, plan.ws_total(), &empty, &zero);
  if (st != kOk || empty) return st;
  if (!plan.fits) return kErrShape;
  if ((st = current_device(nullptr)) != kOk) return st;
  hipStream_t s = (hipStream_t)stream;
  const int oes = g.out_t == 0 ? 2 : 4;
  int64_t out_rows, out_cols;
  if (g.op == kOpFprop || g.op == kOpTensor) {
    out_rows = g.M; out_cols = g.N;
  } else if (g.op == kOpDgrad || g.op == kOpDgradWt) {
    out_rows = g.M; out_cols = g.K;
  } else {
    out_rows = g.N; out_cols = g.K;
  }
  if (zero && g.out_t == 2) return kOk;  // accumulating an empty sum
  if (zero) return launched(launch_zero_fill(const_cast<void*>(g.out), out_rows, out_cols * oes, g.ldout * oes, s));

  GemmDesc d;
  d.c = const_cast<void*>(g.out);
  d.ldc = g.ldout;
  d.out_f32 = g.out_t;
  d.fa = g.fa;
  d.fb = g.fb;
  d.M = out_rows;
  d.N = out_cols;
  d.a = (const uint8_t*)g.qa;
  d.lda = g.ldqa;
  d.sa = (const float*)g.sa;
  d.ldsa = g.ldsa;
  d.sa_mstride = 1;
  d.sb = (const float*)g.sb;
  if (g.op == kOpTensor) {
    // one scale per operand: every scale read of the fprop kernel lands on sa[0] / sb[0]
    d.K = g.K;
    d.b = (const uint8_t*)g.qb;
    d.ldb = g.ldqb;
    d.ldsa = 0;
    d.sa_mstride = 0;
    d.sb_mode = kSbBlock128;
    d.sb_kstride = 0;
    d.sb_nstride = 0;
  } else if (g.op == kOpFprop) {
    d.K = g.K;
    d.b = (const uint8_t*)g.qb;
    d.ldb = g.ldqb;
    d.sb_mode = kSbBlock128;
    d.sb_kstride = 1;          // sw[nb * ldsw + kb]
    d.sb_nstride = g.ldsb;
  } else if (g.op == kOpDgrad) {
    // W[N, K] is read along its rows (contraction over N): transpose the codes once into the
    // workspace so both operands are contiguous along the contraction.
    uint8_t* wt = (uint8_t*)g.ws;
    hipError_t e = launch_transpose_u8((const uint8_t*)g.qb, g.ldqb, wt, g.N, g.N, g.K, s);
    if (e != hipSuccess) return kErrLaunch;
    d.K = g.N;
    d.b = wt;
    d.ldb = g.N;
    d.sb_mode = kSbBlock128;
    d.sb_kstride = g.ldsb;     // sw[nb * ldsw + k / 128]
    d.sb_nstride = 1;
  } else if (g.op == kOpDgradWt) {
    // the caller passes W^T [K, N]: already contiguous along the contraction
    d.K = g.N;
    d.b = (const uint8_t*)g.qb;
    d.ldb = g.ldqb;
    d.sb_mode = kSbBlock128;
    d.sb_kstride = g.ldsb;     // sw[nb * ldsw + k / 128]
    d.sb_nstride = 1;
  } else {
    d.K = g.M;
    d.b = (const uint8_t*)g.qb;
    d.ldb = g.ldqb;
    d.sb_mode = kSbColumn;
    d.sb_kstride = g.ldsb;     // sxt[mb * ldsxt + k]
    d.sb_nstride = 0;
  }
  void* ws_gemm = plan.ws_gemm ? (uint8_t*)g.ws + plan.ws_transpose : nullptr;
  const int kop = g.op == kOpDgradWt ? kOpDgrad : (g.op == kOpTensor ? kOpFprop : g.op);
  return launched(launch_gemm(kop, d, plan, ws_gemm, s));
}

}  // namespace fp8bq

using namespace fp8bq;

extern "C" {

int fp8bq_quantize_act_1x128(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx, fp8bq_fp8 fmt,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
  bool empty = false;
  int st = validate_quant_1x128(x, (int)xt, R, C, ldx, (int)fmt, q, ldq, s, lds, &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_1x128(x, (int)xt, R, C, ldx, (int)fmt, q, ldq, s, lds, (hipStream_t)stream));
}

int fp8bq_quantize_act_128x1(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx, fp8bq_fp8 fmt,
                             uint8_t* qt, int64_t ldqt, float* st_, int64_t ldst, void* stream) {
  bool empty = false;
  int st = validate_quant_128x1(x, (int)xt, R, C, ldx, (int)fmt, qt, ldqt, st_, ldst, &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_128x1(x, (int)xt, R, C, ldx, (int)fmt, qt, ldqt, st_, ldst, (hipStream_t)stream));
}

int fp8bq_quantize_act_dual(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx, fp8bq_fp8 fmt_rows,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds, fp8bq_fp8 fmt_cols, uint8_t* qt,
                            int64_t ldqt, float* st_, int64_t ldst, void* stream) {
  bool empty = false;
  int st = validate_quant_dual(x, (int)xt, R, C, ldx, (int)fmt_rows, q, ldq, s, lds, (int)fmt_cols, qt, ldqt, st_,
                               ldst, &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_dual(x, (int)xt, R, C, ldx, (int)fmt_rows, q, ldq, s, lds, (int)fmt_cols, qt, ldqt,
                                    st_, ldst, (hipStream_t)stream));
}

int fp8bq_quantize_weight_dual(const void* w, fp8bq_in wt, int64_t N, int64_t K, int64_t ldw, fp8bq_fp8 fmt,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                               void* stream) {
  bool empty = false;
  int st = validate_quant_128x128_dual(w, (int)wt, N, K, ldw, (int)fmt, q, ldq, s, lds, qt, ldqt, &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(
      launch_quant_128x128_dual(w, (int)wt, N, K, ldw, (int)fmt, q, ldq, s, lds, qt, ldqt, (hipStream_t)stream));
}

int fp8bq_quantize_weights_dual(const fp8bq_weight_job* jobs, int count, fp8bq_in wt, fp8bq_fp8 fmt,
                                void* stream) {
  static_assert(FP8BQ_MAX_WEIGHT_JOBS == kMaxWeightJobs, "job limit of the header and the launcher");
  WeightJobArgs args[kMaxWeightJobs];
  bool empty[kMaxWeightJobs];
  const int n = (count >= 0 && count <= kMaxWeightJobs && jobs) ? count : 0;
  for (int j = 0; j < n; ++j) {
    const fp8bq_weight_job& a = jobs[j];
    args[j] = WeightJobArgs{a.w, a.N, a.K, a.ldw, a.q, a.ldq, a.s, a.lds, a.qt, a.ldqt};
  }
  int st = validate_quant_weights_dual(n == count ? args : nullptr, count, kMaxWeightJobs, (int)wt, (int)fmt, empty);
  if (st != kOk) return st;
  // one block per 128x128 tile, jobs in order; the grid must stay within 2^31 - 1 blocks
  WeightDualBatch b{};
  uint64_t tiles = 0;
  for (int j = 0; j < count; ++j) {
    if (empty[j]) continue;
    const WeightJobArgs& a = args[j];  // the validated copy, not the caller's array again
    const int i = b.count++;
    b.w[i] = a.w;
    b.q[i] = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.q));
    b.s[i] = const_cast<float*>(static_cast<const float*>(a.s));
    b.qt[i] = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.qt));
    b.ldw[i] = a.ldw; b.ldq[i] = a.ldq; b.lds[i] = a.lds; b.ldqt[i] = a.ldqt;
    b.nkb[i] = (uint32_t)(a.K / 128);
    b.start[i] = (uint32_t)tiles;
    tiles += (uint64_t)(a.N / 128) * (uint64_t)(a.K / 128);
    if (tiles > 0x7fffffffull) return kErrShape;
  }
  b.start[b.count] = (uint32_t)tiles;
  if (b.count == 0) return kOk;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_weights_dual(b, (int)wt, (int)fmt, (hipStream_t)stream));
}

int fp8bq_quantize_weight_128x128(const void* w, fp8bq_in wt, int64_t N, int64_t K, int64_t ldw, fp8bq_fp8 fmt,
                                  uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
  bool empty = false;
  int st = validate_quant_128x128(w, (int)wt, N, K, ldw, (int)fmt, q, ldq, s, lds, &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_128x128(w, (int)wt, N, K, ldw, (int)fmt, q, ldq, s, lds, (hipStream_t)stream));
}

int fp8bq_gemm_fprop(int64_t M, int64_t N, int64_t K, const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx,
                     fp8bq_fp8 fx, const uint8_t* qw, int64_t ldqw, const float* sw, int64_t ldsw, fp8bq_fp8 fw,
                     void* y, fp8bq_out yt, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  GemmArgs g{kOpFprop, M, N, K, qx, ldqx, sx, ldsx, (int)fx, qw, ldqw, sw, ldsw, (int)fw, y, (int)yt, ldy, ws,
             ws_bytes};
  return run_gemm(g, stream);
}

int fp8bq_gemm_dgrad(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, int64_t ldqdy, const float* sdy,
                     int64_t ldsdy, fp8bq_fp8 fdy, const uint8_t* qw, int64_t ldqw, const float* sw, int64_t ldsw,
                     fp8bq_fp8 fw, void* dx, fp8bq_out dxt, int64_t lddx, void* ws, size_t ws_bytes, void* stream) {
  GemmArgs g{kOpDgrad, M, N, K, qdy, ldqdy, sdy, ldsdy, (int)fdy, qw, ldqw, sw, ldsw, (int)fw, dx, (int)dxt, lddx,
             ws, ws_bytes};
  return run_gemm(g, stream);
}

int fp8bq_gemm_dgrad_wt(int64_t M, int64_t N, int64_t K, const uint8_t* qdy, int64_t ldqdy, const float* sdy,
                        int64_t ldsdy, fp8bq_fp8 fdy, const uint8_t* qwt, int64_t ldqwt, const float* sw,
                        int64_t ldsw, fp8bq_fp8 fw, void* dx, fp8bq_out dxt, int64_t lddx, void* ws, size_t ws_bytes,
                        void* stream) {
  GemmArgs g{kOpDgradWt, M, N, K, qdy, ldqdy, sdy, ldsdy, (int)fdy, qwt, ldqwt, sw, ldsw, (int)fw, dx, (int)dxt,
             lddx, ws, ws_bytes};
  return run_gemm(g, stream);
}

int fp8bq_gemm_wgrad(int64_t M, int64_t N, int64_t K, const uint8_t* qdyt, int64_t ldqdyt, const float* sdyt,
                     int64_t ldsdyt, fp8bq_fp8 fdy, const uint8_t* qxt, int64_t ldqxt, const float* sxt,
                     int64_t ldsxt, fp8bq_fp8 fx, void* dw, fp8bq_out dwt, int64_t lddw, void* ws, size_t ws_bytes,
                     void* stream) {
  GemmArgs g{kOpWgrad, M, N, K, qdyt, ldqdyt, sdyt, ldsdyt, (int)fdy, qxt, ldqxt, sxt, ldsxt, (int)fx, dw, (int)dwt,
             lddw, ws, ws_bytes};
  return run_gemm(g, stream);
}

int fp8bq_gemm_tensor(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t ldqa, const float* sa,
                      fp8bq_fp8 fa, const uint8_t* qb, int64_t ldqb, const float* sb, fp8bq_fp8 fb, void* out,
                      fp8bq_out out_t, int64_t ldout, void* ws, size_t ws_bytes, void* stream) {
  GemmArgs g{kOpTensor, M, N, K, qa, ldqa, sa, 1, (int)fa, qb, ldqb, sb, 1, (int)fb, out, (int)out_t, ldout, ws,
             ws_bytes};
  return run_gemm(g, stream);
}

size_t fp8bq_quantize_tensor_workspace_size(int64_t R, int64_t C) {
  if (R <= 0 || C <= 0) return 0;
  return kTensorWorkspace;
}

int fp8bq_quantize_tensor_delayed(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx, fp8bq_fp8 fmt,
                                  float* amax, double beta, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                  float* s, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  int st = validate_quant_tensor(x, (int)xt, R, C, ldx, (int)fmt, amax, beta, q, ldq, qt, ldqt, s, ws, ws_bytes,
                                 fp8bq_quantize_tensor_workspace_size(R, C), &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_quant_tensor_delayed(x, (int)xt, R, C, ldx, (int)fmt, amax, beta, q, ldq, qt, ldqt, s, ws,
                                              (hipStream_t)stream));
}

int fp8bq_quantize_tensor_delayed_noalloc(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx,
                                          fp8bq_fp8 fmt, float* amax, double beta, uint8_t* q, int64_t ldq,
                                          uint8_t* qt, int64_t ldqt, float* s, void* stream) {
  bool empty = false;
  int st = validate_quant_tensor(x, (int)xt, R, C, ldx, (int)fmt, amax, beta, q, ldq, qt, ldqt, s, nullptr, 0, 0,
                                 &empty);
  if (st != kOk || empty) return st;
  int dev = -1;
  if ((st = current_device(nullptr, &dev)) != kOk) return st;
  float* scr = nullptr;
  if (tensor_scratch(dev, &scr) != hipSuccess) {
    (void)hipGetLastError();
    return kErrDevice;
  }
  return launched(launch_quant_tensor_delayed(x, (int)xt, R, C, ldx, (int)fmt, amax, beta, q, ldq, qt, ldqt, s, scr,
                                              (hipStream_t)stream));
}

size_t fp8bq_hyperball_workspace_size(int64_t R, int64_t C) {
  if (R <= 0 || C <= 0) return 0;
  return kHyperballWorkspace;
}

int fp8bq_hyperball_step(float* w, int64_t ldw, const void* g, fp8bq_in gt, int64_t ldg, int64_t R, int64_t C,
                         double lr, double weight_decay, double eps, double radius, float* norms, void* ws,
                         size_t ws_bytes, void* stream) {
  bool empty = false;
  int st = validate_hyperball(w, ldw, g, (int)gt, ldg, R, C, lr, weight_decay, eps, radius, norms, ws, ws_bytes,
                              fp8bq_hyperball_workspace_size(R, C), &empty);
  if (st != kOk || empty) return st;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_hyperball_step(w, ldw, g, (int)gt, ldg, R, C, lr, weight_decay, eps, radius, norms, ws,
                                        (hipStream_t)stream));
}

size_t fp8bq_hyperball_batch_workspace_size(int count) {
  return (count < 0 || count > kMaxHyperballJobs) ? 0 : (size_t)count * kHyperballWorkspace;
}

int fp8bq_hyperball_step_batch(const fp8bq_hyperball_job* jobs, int count, fp8bq_in gt, double lr,
                               double weight_decay, double eps, void* ws, size_t ws_bytes, void* stream) {
  static_assert(FP8BQ_MAX_HYPERBALL_JOBS == kMaxHyperballJobs, "batch limit");
  HyperballJobArgs a[kMaxHyperballJobs];
  bool empty[kMaxHyperballJobs] = {};
  const int n = (count >= 0 && count <= kMaxHyperballJobs) ? count : 0;
  for (int j = 0; j < n; ++j)
    a[j] = HyperballJobArgs{jobs ? jobs[j].w : nullptr, jobs ? jobs[j].ldw : 0, jobs ? jobs[j].g : nullptr,
                            jobs ? jobs[j].ldg : 0, jobs ? jobs[j].R : 0, jobs ? jobs[j].C : 0,
                            jobs ? jobs[j].radius : 0.0, jobs ? jobs[j].norms : nullptr};
  int st = validate_hyperball_batch(jobs ? a : nullptr, count, kMaxHyperballJobs, (int)gt, lr, weight_decay, eps, ws,
                                    ws_bytes, fp8bq_hyperball_batch_workspace_size(count), empty);
  if (st != kOk) return st;
  HyperballBatch b{};
  b.partial = reinterpret_cast<double*>(ws);
  uint32_t blocks = 0;
  for (int j = 0; j < count; ++j) {
    if (empty[j]) continue;
    const int k = b.count++;
    b.w[k] = jobs[j].w;
    b.g[k] = jobs[j].g;
    b.ldw[k] = jobs[j].ldw;
    b.ldg[k] = jobs[j].ldg;
    b.R[k] = jobs[j].R;
    b.C[k] = jobs[j].C;
    b.radius[k] = jobs[j].radius;
    b.norms[k] = jobs[j].norms;
    b.start[k] = blocks;
    blocks += (uint32_t)hyperball_blocks(jobs[j].R);
  }
  if (b.count == 0) return kOk;
  b.start[b.count] = blocks;
  if ((st = current_device(nullptr)) != kOk) return st;
  return launched(launch_hyperball_batch(b, (int)gt, lr, weight_decay, eps, (hipStream_t)stream));
}

int fp8bq_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  bool empty = false;
  int st = validate_stream_copy(src, dst, bytes, &empty);
  if (st != kOk || empty) return st;
  int cus = 0;
  if ((st = current_device(&cus)) != kOk) return st;
  return launched(launch_stream_copy(src, dst, bytes, cus, (hipStream_t)stream));
}

size_t fp8bq_gemm_workspace_size(fp8bq_op op, int64_t M, int64_t N, int64_t K) {
  if ((int)op < 0 || (int)op > 4 || M < 0 || N < 0 || K < 0) return 0;
  return plan_gemm((int)op, M, N, K, cu_count_or_default()).ws_total();
}

int fp8bq_gemm_plan(fp8bq_op op, int64_t M, int64_t N, int64_t K, int32_t* tile_m, int32_t* tile_n,
                    int32_t* split_k) {
  if (!tile_m || !tile_n || !split_k) return kErrNull;
  if ((int)op < 0 || (int)op > 4 || M < 0 || N < 0 || K < 0) return kErrShape;
  const GemmPlan p = plan_gemm((int)op, M, N, K, cu_count_or_default());
  if (!p.fits) return kErrShape;
  *tile_m = p.tile_m;
  *tile_n = p.tile_n;
  *split_k = p.split_k;
  return kOk;
}

const char* fp8bq_status_string(int status) {
  switch (status) {
    case kOk: return "FP8BQ_OK";
    case kErrNull: return "FP8BQ_ERR_NULL: a required pointer is NULL";
    case kErrShape: return "FP8BQ_ERR_SHAPE: negative size or a grouped/contracted size not a multiple of 128";
    case kErrLd: return "FP8BQ_ERR_LD: leading dimension too small, misaligned, or too large for a code operand";
    case kErrAlign: return "FP8BQ_ERR_ALIGN: pointer not 16-byte aligned";
    case kErrDtype: return "FP8BQ_ERR_DTYPE: unknown element type";
    case kErrFormat: return "FP8BQ_ERR_FORMAT: unknown FP8 format";
    case kErrWorkspace: return "FP8BQ_ERR_WORKSPACE: workspace missing or too small";
    case kErrDevice: return "FP8BQ_ERR_DEVICE: no current HIP device or it is not gfx950";
    case kErrLaunch: return "FP8BQ_ERR_LAUNCH: kernel launch failed";
    case kErrOverlap: return "FP8BQ_ERR_OVERLAP: an output overlaps an input";
    case kErrValue: return "FP8BQ_ERR_VALUE: a scalar argument is out of range or not finite";
    default: return "FP8BQ_ERR_UNKNOWN";
  }
}

int fp8bq_version(void) { return 100; }

}  // extern "C"
