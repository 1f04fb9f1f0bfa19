/*
 * fp8bq.h -- FP8 blockwise-quantized linear layer for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of the Puro-2B FP8 recipe:
 *   - "用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析" (hankli.space),
 *     section "Blackwell 的 FP8 Tensor Core" (the E4M3 / E5M2 formats, maxima 448 and 57344)
 *     and section "核心挑战：Scale Factor 管理" (FP8Linear: scale = amax / fmt_max with a
 *     1e-12 floor, divide, clamp to +-fmt_max, cast; dequantize = code value * scale);
 *   - "小团队也能预训练！普罗2B：RTX5090训练成本不到5090美元" (66bd.net), paragraph
 *     "FP8发挥RTX 5090的低精度效率优势" (DeepSeek-V3-style fine-grained blocks, linear GEMMs in
 *     FP8, sensitive state in BF16/FP32);
 *   - "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090" (AI Papers Daily),
 *     section "方法关键点", bullet "FP8 blockwise 混合精度" (E4M3 linear GEMMs, activations in
 *     groups of 128, weights in 128x128 blocks).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The library never frees,
 *   retains or allocates caller memory; callers provide any workspace.
 * - Matrices are row-major.  Sizes and leading dimensions (ld*) are in ELEMENTS.
 * - Each call validates all arguments first; on any argument error it returns a nonzero
 *   fp8bq_status and enqueues nothing.  On success it enqueues its kernels on `stream` (a
 *   hipStream_t; NULL means the default stream) and returns FP8BQ_OK without synchronizing.  Faults
 *   on the device surface at the caller's next synchronization, as usual for HIP.  A call that
 *   launches several kernels checks each launch (hipGetLastError, which also clears the thread's
 *   last HIP error) and stops at the first that fails, returning FP8BQ_ERR_LAUNCH: the kernels
 *   launched before it stay enqueued.
 * - Outputs are fully overwritten, with three documented exceptions that update caller memory in
 *   place: FP8BQ_OUT_F32_ACCUM (fp8bq_gemm_wgrad adds its result to the FP32 output), the running
 *   amax of fp8bq_quantize_tensor_delayed[_noalloc] (read and updated), and the weights of
 *   fp8bq_hyperball_step and fp8bq_hyperball_step_batch (read and updated).
 * - Calls are thread-safe and re-entrant; there is no mutable global state besides a per-device
 *   cache of the device's architecture check.  Calls that write overlapping outputs on the same
 *   device must be ordered by the caller (same stream or events).
 * - Alignment: every tensor pointer must be 16-byte aligned, and each leading dimension times
 *   the element size must be a multiple of 16 bytes (bf16: ld % 8 == 0; fp32: ld % 4 == 0;
 *   codes: ld % 16 == 0).  Scale arrays follow the same rule (ld % 4 == 0).
 * - Inputs must be finite; NaN or Inf inputs give unspecified codes.
 * - A dimension of size 0 makes the call a successful no-op.
 *
 * Quantization rule (per group of values, identical for all three quantizers):
 *   amax = max |x|;  s = max(fp32(amax / fmt_max), fp32(1e-12));
 *   q = round-to-nearest-even FP8 code of clamp(fp32(x / s), -fmt_max, fmt_max)
 * where both divisions are IEEE fp32 divisions rounded to nearest even and the sign of a
 * value that rounds to zero is kept.  Codes and scales are a deterministic function of the
 * input: they are bit-identical from call to call.  Dequantized value = decode(q) * s.
 */
#ifndef FP8BQ_H_
#define FP8BQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BQ_OK = 0,
  FP8BQ_ERR_NULL = 1,      /* a required pointer is NULL */
  FP8BQ_ERR_SHAPE = 2,     /* negative size, a grouped/contracted size not a multiple of 128, a
                              matrix spanning 2^48 bytes or more, or a GEMM with 2^28 or more
                              output tiles of 128x128 */
  FP8BQ_ERR_LD = 3,        /* leading dimension smaller than the row length, or misaligned; for the
                              GEMMs' code operands also 255 * ld + contraction length >= 2^32 bytes
                              (a 256-row tile is addressed through a 32-bit range: rows of codes
                              up to about 16.8 MB) */
  FP8BQ_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  FP8BQ_ERR_DTYPE = 5,     /* unknown input or output element type */
  FP8BQ_ERR_FORMAT = 6,    /* unknown FP8 format */
  FP8BQ_ERR_WORKSPACE = 7, /* workspace NULL or smaller than fp8bq_gemm_workspace_size() */
  FP8BQ_ERR_DEVICE = 8,    /* no current HIP device, or it is not gfx950 */
  FP8BQ_ERR_LAUNCH = 9,    /* the kernel launch itself failed */
  FP8BQ_ERR_OVERLAP = 10,  /* an output overlaps an input the same call reads */
  FP8BQ_ERR_VALUE = 11     /* a scalar argument is out of range or not finite */
} fp8bq_status;

/* OCP FP8 formats: E4M3 = float8_e4m3fn (bias 7, no Inf, max 448);
 * E5M2 = float8_e5m2 (bias 15, IEEE-like Inf/NaN, max 57344). */
typedef enum { FP8BQ_E4M3 = 0, FP8BQ_E5M2 = 1 } fp8bq_fp8;

/* Element type of a high-precision input. */
typedef enum { FP8BQ_IN_BF16 = 0, FP8BQ_IN_F32 = 1 } fp8bq_in;

/* Element type of a GEMM output: BF16 (round to nearest even from the FP32 accumulator), or
 * FP32 (the accumulator itself).  FP8BQ_OUT_F32_ACCUM (fp8bq_gemm_wgrad only) adds the FP32
 * result to the FP32 values already in the output, for a main-grad buffer kept in FP32 across
 * micro-batches: out = fp32(out + result).  The pages keep precision-sensitive state in BF16/FP32
 * while the linear GEMMs run in FP8 ("Puro-2B" summary, method key points: FP8 blockwise mixed
 * precision). */
typedef enum { FP8BQ_OUT_BF16 = 0, FP8BQ_OUT_F32 = 1, FP8BQ_OUT_F32_ACCUM = 2 } fp8bq_out;

/* GEMM selector for fp8bq_gemm_workspace_size and fp8bq_gemm_plan (FP8BQ_OP_DGRAD_WT:
 * fp8bq_gemm_dgrad_wt; FP8BQ_OP_TENSOR: fp8bq_gemm_tensor). */
typedef enum {
  FP8BQ_OP_FPROP = 0,
  FP8BQ_OP_DGRAD = 1,
  FP8BQ_OP_WGRAD = 2,
  FP8BQ_OP_DGRAD_WT = 3,
  FP8BQ_OP_TENSOR = 4
} fp8bq_op;

/*
 * Activation quantization, one scale per 1x128 group (128 consecutive elements of a row).
 * Defining passages: the quantize rule of FP8Linear (hankli.space, "核心挑战：Scale Factor 管理");
 * the 1-D groups of 128 for activations (AI Papers Daily, "FP8 blockwise 混合精度").
 *
 *   x  [R, C]  input, element type xt, row stride ldx (>= C).  C % 128 == 0; R >= 0 is free.
 *   q  [R, C]  output codes (uint8), row stride ldq (>= C).
 *   s  [C/128][R] output scales (fp32), group-major: the scale of row r, group g is s[g*lds + r]
 *              (lds >= R).  This layout makes the scales of one 128-wide contraction block
 *              contiguous over rows, which is how the GEMMs read them.
 * Used for X before fprop and for dY before dgrad.
 */
int fp8bq_quantize_act_1x128(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx,
                             fp8bq_fp8 fmt, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             void* stream);

/*
 * Activation quantization along the token axis, one scale per 128x1 group (128 consecutive
 * ROWS of one column), quantized from the original x (not from 1x128 codes), with transposed
 * outputs so that the token axis is contiguous.  This is the same 1-D group of 128 laid along
 * the axis wgrad contracts over (fine-grained blocks after DeepSeek-V3: 66bd.net,
 * "FP8发挥RTX 5090的低精度效率优势"; rule as above).
 *
 *   x  [R, C]  input, element type xt, row stride ldx (>= C).  R % 128 == 0; C % 8 == 0.
 *   qt [C, R]  output codes transposed: qt[c*ldqt + r] is the code of x[r, c] (ldqt >= R).
 *   st [R/128][C] output scales: the scale of rows 128*rb .. 128*rb+127 of column c is
 *              st[rb*ldst + c] (ldst >= C).
 * Used for X and dY before wgrad.
 */
int fp8bq_quantize_act_128x1(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx,
                             fp8bq_fp8 fmt, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                             void* stream);

/*
 * Weight quantization with a transposed copy of the codes, from one read of w: q and s exactly as
 * fp8bq_quantize_weight_128x128, plus qt [K, N] with qt[k*ldqt + n] = q[n*ldq + k] (ldqt >= N,
 * ldqt % 16 == 0), the operand layout of fp8bq_gemm_dgrad_wt.  N % 128 == 0; K % 128 == 0.  No
 * output may overlap w or another output.  Defining passages: as fp8bq_quantize_weight_128x128.
 */
int fp8bq_quantize_weight_dual(const void* w, fp8bq_in wt, int64_t N, int64_t K, int64_t ldw, fp8bq_fp8 fmt,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt,
                               void* stream);

/* One weight of fp8bq_quantize_weights_dual: the arguments fp8bq_quantize_weight_dual takes for it. */
typedef struct {
  const void* w;   /* [N, K], row stride ldw */
  int64_t N, K, ldw;
  uint8_t* q;      /* [N, K] codes, row stride ldq */
  int64_t ldq;
  float* s;        /* [N/128][K/128] scales, row stride lds */
  int64_t lds;
  uint8_t* qt;     /* [K, N] transposed codes, row stride ldqt */
  int64_t ldqt;
} fp8bq_weight_job;

#define FP8BQ_MAX_WEIGHT_JOBS 16

/*
 * Several weights quantized in one launch.  For each of the count jobs (jobs is a HOST array, read
 * only during the call; 0 <= count <= FP8BQ_MAX_WEIGHT_JOBS, else FP8BQ_ERR_VALUE) the outputs are
 * exactly those of fp8bq_quantize_weight_dual(job.w, wt, job.N, job.K, job.ldw, fmt, job.q, job.ldq,
 * job.s, job.lds, job.qt, job.ldqt), bit for bit.  All weights share the input type wt and the format
 * fmt.  Every job must pass that call's checks (a job with N or K equal to 0 is skipped); besides, no
 * job's outputs may overlap another job's input or outputs (FP8BQ_ERR_OVERLAP), while inputs may be
 * shared.  The jobs' 128x128 tiles together must number under 2^31 (FP8BQ_ERR_SHAPE).  On error the
 * first failing check's status is returned and nothing is enqueued.
 * In a training step every weight is known at its start; one launch for all of them keeps the GPU
 * busy where one weight alone is too small to fill it.  Defining passages: as
 * fp8bq_quantize_weight_128x128.
 */
int fp8bq_quantize_weights_dual(const fp8bq_weight_job* jobs, int count, fp8bq_in wt, fp8bq_fp8 fmt,
                                void* stream);

/*
 * Both activation layouts from one read of x: the outputs of
 *   fp8bq_quantize_act_1x128(x, xt, R, C, ldx, fmt_rows, q, ldq, s, lds) and
 *   fp8bq_quantize_act_128x1(x, xt, R, C, ldx, fmt_cols, qt, ldqt, st, ldst),
 * bit for bit, for about two thirds of their combined memory traffic.  A layer quantizes its
 * input X both ways (fprop, wgrad) and its output gradient dY both ways (dgrad, wgrad); the two
 * formats are independent (e.g. E5M2 for dgrad's dY, E4M3 for wgrad's).  Defining passages: as the
 * two quantizers above.
 *
 *   x  [R, C]  input, element type xt, row stride ldx (>= C).  R % 128 == 0; C % 128 == 0.
 *   q, s       as fp8bq_quantize_act_1x128 (q [R, C], s [C/128][R]).
 *   qt, st     as fp8bq_quantize_act_128x1 (qt [C, R], st [R/128][C]).
 * No output may overlap x or another output (FP8BQ_ERR_OVERLAP).
 */
int fp8bq_quantize_act_dual(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx,
                            fp8bq_fp8 fmt_rows, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            fp8bq_fp8 fmt_cols, uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                            void* stream);

/*
 * Weight quantization, one scale per aligned 128x128 tile.
 * Defining passages: FP8Linear's rule (hankli.space, "核心挑战：Scale Factor 管理"); 2-D
 * 128x128 blocks for weights (AI Papers Daily, "FP8 blockwise 混合精度").
 *
 *   w  [N, K]  input, element type wt, row stride ldw (>= K).  N % 128 == 0, K % 128 == 0.
 *   q  [N, K]  output codes, row stride ldq (>= K).
 *   s  [N/128][K/128] output scales: tile (nb, kb) has scale s[nb*lds + kb] (lds >= K/128).
 * The same codes and scales serve fprop (W) and dgrad (W read along its rows).
 */
int fp8bq_quantize_weight_128x128(const void* w, fp8bq_in wt, int64_t N, int64_t K, int64_t ldw,
                                  fp8bq_fp8 fmt, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                  void* stream);

/*
 * Forward GEMM  Y[M, N] = X[M, K] . W[N, K]^T  on FP8 operands with per-block scales,
 * FP32 accumulation and BF16 (or FP32) output:
 *   Y[m, n] = sum_kb sx(m, kb) * sw(n/128, kb) * sum_{k in kb} dec(qx[m, k]) * dec(qw[n, k]).
 * Defining passages: linear-layer GEMMs in FP8 with high-precision accumulation and state
 * (66bd.net, "FP8发挥RTX 5090的低精度效率优势"; AI Papers Daily, "FP8 blockwise 混合精度");
 * dequantize-then-contract as in FP8Linear.forward (hankli.space).
 *
 *   qx/sx  from fp8bq_quantize_act_1x128(X): qx [M, K] (ldqx), sx [K/128][M] (ldsx >= M).
 *   qw/sw  from fp8bq_quantize_weight_128x128(W): qw [N, K] (ldqw), sw [N/128][K/128] (ldsw).
 *   fx/fw  the FP8 format of each operand (any combination of E4M3 / E5M2).
 *   y      [M, N] output of type yt, row stride ldy (>= N).
 *   M >= 0 is free; N % 128 == 0; K % 128 == 0.
 *   ws/ws_bytes  device workspace of at least fp8bq_gemm_workspace_size(FP8BQ_OP_FPROP, M, N, K)
 *          bytes (may be NULL when that size is 0).  Its contents are scratch.
 */
int fp8bq_gemm_fprop(int64_t M, int64_t N, int64_t K,
                     const uint8_t* qx, int64_t ldqx, const float* sx, int64_t ldsx, fp8bq_fp8 fx,
                     const uint8_t* qw, int64_t ldqw, const float* sw, int64_t ldsw, fp8bq_fp8 fw,
                     void* y, fp8bq_out yt, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/*
 * Data-gradient GEMM  dX[M, K] = dY[M, N] . W[N, K]  (contraction over the N output features):
 *   dX[m, k] = sum_nb sdy(m, nb) * sw(nb, k/128) * sum_{n in nb} dec(qdy[m, n]) * dec(qw[n, k]).
 * Defining passages: as fprop (all linear GEMMs of the layer run in FP8); gradients may use
 * E5M2 (hankli.space, "Blackwell 的 FP8 Tensor Core").
 *
 *   qdy/sdy  from fp8bq_quantize_act_1x128(dY): qdy [M, N] (ldqdy), sdy [N/128][M] (ldsdy >= M).
 *   qw/sw    the weight's codes and scales exactly as produced for fprop.
 *   dx       [M, K] output of type dxt, row stride lddx (>= K).
 *   M >= 0 is free; N % 128 == 0; K % 128 == 0.
 *   ws       at least fp8bq_gemm_workspace_size(FP8BQ_OP_DGRAD, M, N, K) bytes (holds W's codes
 *            transposed to [K, N] for the duration of the call).
 */
int fp8bq_gemm_dgrad(int64_t M, int64_t N, int64_t K,
                     const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy, fp8bq_fp8 fdy,
                     const uint8_t* qw, int64_t ldqw, const float* sw, int64_t ldsw, fp8bq_fp8 fw,
                     void* dx, fp8bq_out dxt, int64_t lddx, void* ws, size_t ws_bytes, void* stream);

/*
 * dgrad with the weight codes already transposed: the result of fp8bq_gemm_dgrad, computed from
 * qwt [K, N] (ldqwt >= N), the W^T codes of fp8bq_quantize_weight_dual, instead of qw.  No
 * transpose runs, so the workspace holds only split partial sums:
 * fp8bq_gemm_workspace_size(FP8BQ_OP_DGRAD_WT, M, N, K) bytes (often 0; ws may then be NULL).
 * Other arguments as fp8bq_gemm_dgrad (sw: the weight scales, [N/128][K/128]).
 */
int fp8bq_gemm_dgrad_wt(int64_t M, int64_t N, int64_t K,
                        const uint8_t* qdy, int64_t ldqdy, const float* sdy, int64_t ldsdy, fp8bq_fp8 fdy,
                        const uint8_t* qwt, int64_t ldqwt, const float* sw, int64_t ldsw, fp8bq_fp8 fw,
                        void* dx, fp8bq_out dxt, int64_t lddx, void* ws, size_t ws_bytes, void* stream);

/*
 * Weight-gradient GEMM  dW[N, K] = dY[M, N]^T . X[M, K]  (contraction over the M tokens):
 *   dW[n, k] = sum_mb sdy(mb, n) * sx(mb, k) * sum_{m in mb} dec(qdy[m, n]) * dec(qx[m, k]).
 * Defining passages: as fprop; both operands carry 128x1 (token-axis) scales, an outer product
 * per 128-token block.
 *
 *   qdyt/sdyt  from fp8bq_quantize_act_128x1(dY): qdyt [N, M] (ldqdyt >= M), sdyt [M/128][N].
 *   qxt/sxt    from fp8bq_quantize_act_128x1(X):  qxt [K, M] (ldqxt >= M),  sxt [M/128][K].
 *   dw         [N, K] output of type dwt, row stride lddw (>= K).  With FP8BQ_OUT_F32_ACCUM, dw
 *              holds FP32 values on entry and receives dw + dW (a zero-length contraction, M == 0,
 *              leaves it unchanged); the other GEMMs reject that type with FP8BQ_ERR_DTYPE.
 *   M % 128 == 0; N % 128 == 0; K % 128 == 0.
 *   ws         at least fp8bq_gemm_workspace_size(FP8BQ_OP_WGRAD, M, N, K) bytes (FP32 partial
 *              sums when the contraction is split across workgroups).
 */
int fp8bq_gemm_wgrad(int64_t M, int64_t N, int64_t K,
                     const uint8_t* qdyt, int64_t ldqdyt, const float* sdyt, int64_t ldsdyt, fp8bq_fp8 fdy,
                     const uint8_t* qxt, int64_t ldqxt, const float* sxt, int64_t ldsxt, fp8bq_fp8 fx,
                     void* dw, fp8bq_out dwt, int64_t lddw, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-tensor delayed scaling: the pages' own alternative to the blockwise recipe.
 * Defining passage: "用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析", section
 * "核心挑战：Scale Factor 管理", the FP8Linear listing (_update_amax, _quantize, forward): one scale
 * per tensor from a running amax that is updated before the tensor is quantized.
 *
 * fp8bq_quantize_tensor_delayed, for x [R, C] (row-major, ldx >= C):
 *   1. cur = max |x| over the whole tensor, of the values as given (BF16 or FP32);
 *   2. fresh = fp32(cur * fp32(1 - beta)), 1 - beta formed in double, and for a BF16 tensor
 *      rounded to BF16 (nearest, ties to even): the listing weights the current amax in the
 *      tensor's own type;  *amax = fp32(fp32(*amax * fp32(beta)) + fresh).  The listing uses
 *      beta = 0.99 and starts the running amax at 1.0;
 *   3. *s = max(fp32(*amax / fmt_max), fp32(1e-12));
 *   4. q[r, c] = RNE code of clamp(fp32(bf16(x[r, c]) / *s), +-fmt_max): the codes of x's BF16
 *      copy (identical to x for BF16 input); and, if qt is not NULL, qt[c, r] = q[r, c] (the
 *      operand layout of dgrad and wgrad).
 *   amax, s    device pointers to one float each (4-byte aligned); *amax is read and updated in
 *              place, *s is written.  Calls that share an amax buffer must be ordered (one stream).
 *   q          [R, C] codes (ldq >= C); qt NULL or [C, R] codes (ldqt >= R, R % 128 == 0).
 *   C % 128 == 0; R >= 0.  R == 0 or C == 0: nothing is enqueued and *amax, *s stay as they are.
 *   ws         at least fp8bq_quantize_tensor_workspace_size(R, C) bytes, 16-byte aligned
 *              (per-block partial maxima; its contents are not needed between calls).
 * Errors: FP8BQ_ERR_VALUE for beta outside [0, 1] (or NaN); FP8BQ_ERR_ALIGN for amax or s not
 * 4-byte aligned; otherwise as the blockwise quantizers.  Two kernels run on `stream` in order:
 * the partial maxima, then the codes (every block derives the scale from the partials; the first
 * also stores the new running amax and the scale).
 */
size_t fp8bq_quantize_tensor_workspace_size(int64_t R, int64_t C);
int fp8bq_quantize_tensor_delayed(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx, fp8bq_fp8 fmt,
                                  float* amax, double beta, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                  float* s, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8bq_quantize_tensor_delayed without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Outputs, running-amax update and errors are exactly those of
 * fp8bq_quantize_tensor_delayed (minus FP8BQ_ERR_WORKSPACE); the kernels use the library's own
 * scratch instead: a fixed fp8bq_quantize_tensor_workspace_size() bytes (4352) of device memory per
 * GPU, held from the first call on that GPU until the process ends, enough for any R and C.  The
 * call allocates nothing.  Every call on one GPU shares that scratch, so calls that may overlap on
 * one GPU (other streams, other host threads) race: order them (one stream, or events).  Nothing in
 * the scratch needs clearing between calls.  FP8BQ_ERR_DEVICE also if the scratch's device address
 * cannot be obtained.
 */
int fp8bq_quantize_tensor_delayed_noalloc(const void* x, fp8bq_in xt, int64_t R, int64_t C, int64_t ldx,
                                          fp8bq_fp8 fmt, float* amax, double beta, uint8_t* q, int64_t ldq,
                                          uint8_t* qt, int64_t ldqt, float* s, void* stream);

/*
 * GEMM of two per-tensor-scaled operands, both contiguous along the contraction ("TN"):
 *   out[m, n] = (*sa) * (*sb) * sum_k dec(qa[m, k]) * dec(qb[n, k]),  FP32 accumulation.
 * Defining passage: as fp8bq_quantize_tensor_delayed (the listing's forward dequantizes both
 * operands with their scales and contracts; its production note runs that product as an FP8 GEMM).
 * fprop: qa = X codes [M, K], qb = W codes [N, K]; dgrad: qa = dY codes [M, N], qb = W^T codes
 * (qt of the weight) with K and N swapped; wgrad: qa = dY^T codes, qb = X^T codes (the qt outputs),
 * contraction over the tokens.
 *   sa, sb     device pointers to one float each (4-byte aligned).
 *   M >= 0 (any); N % 128 == 0; K % 128 == 0; out [M, N] of type out_t (BF16 or FP32), ldout >= N.
 *   ws         at least fp8bq_gemm_workspace_size(FP8BQ_OP_TENSOR, M, N, K) bytes.
 * Errors as fp8bq_gemm_fprop.
 */
int fp8bq_gemm_tensor(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t ldqa, const float* sa,
                      fp8bq_fp8 fa, const uint8_t* qb, int64_t ldqb, const float* sb, fp8bq_fp8 fb, void* out,
                      fp8bq_out out_t, int64_t ldout, void* ws, size_t ws_bytes, void* stream);

/*
 * Hyperball normalized update of one weight matrix, in place, with the optional fixed-radius
 * projection.
 * Defining passages: "用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析", section
 * "Hyperball 优化：让 FP8 训练不爆炸" (HyperballSGD: only the gradient's direction is used, with
 * decoupled weight decay); "小团队也能预训练！普罗2B：RTX5090训练成本不到5090美元", MuonH paragraph, and
 * "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090", section "方法关键点" (MuonH:
 * after the update the weight is projected back onto a fixed radius).
 *
 *   n = max(||g||_2, eps);  w <- fp32(w * fp32(1 - lr*wd)) + fp32(g * fp32(-lr / n));
 *   if radius > 0 and ||w||_F > 0:  w <- fp32(w * fp32(radius / ||w||_F)).
 * Norms are summed in fp64 over fixed per-block partials (deterministic).
 *   w       [R, C] FP32 master weights (ldw >= C), read and written.
 *   g       [R, C] gradient, BF16 or FP32 (gt), ldg >= C; for example dW from fp8bq_gemm_wgrad.
 *   C % 8 == 0.  R == 0 or C == 0: nothing is enqueued.
 *   lr >= 0, weight_decay >= 0, eps > 0, radius >= 0 (0: no projection), all finite; else
 *           FP8BQ_ERR_VALUE.  The pages' defaults are lr 1e-4, weight_decay 0.1, eps 1e-8.
 *   norms   NULL, or two device floats (4-byte aligned) that receive ||g||_2 (before the clamp) and
 *           ||w||_F after the update and before the projection.
 *   ws      at least fp8bq_hyperball_workspace_size(R, C) bytes, 16-byte aligned.
 * w may not overlap g, ws or norms (FP8BQ_ERR_OVERLAP).  Two sweeps run on `stream` in order: the
 * sums of g*g (and, with a radius or norms, of w*w and w*g); then the update, which writes w once:
 * each block reduces those sums to the step coefficient and, with a radius, to the projection
 * factor, ||w'||^2 being d^2 sum w^2 + 2 d c sum wg + c^2 sum g^2 for the FP32 factors
 * d = fp32(1 - lr*wd) and c = fp32(-lr/n) that the update applies.
 */
size_t fp8bq_hyperball_workspace_size(int64_t R, int64_t C);
int fp8bq_hyperball_step(float* w, int64_t ldw, const void* g, fp8bq_in gt, int64_t ldg, int64_t R, int64_t C,
                         double lr, double weight_decay, double eps, double radius, float* norms, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Several Hyperball steps in one launch pair, for many weight matrices (callers that update a model
 * layer by layer would otherwise pay two launches per matrix).  Each job is exactly one
 * fp8bq_hyperball_step call: same rule, same per-matrix norms, and bit-identical weights and norms
 * (the same block decomposition and reduction order per matrix).  Defining passages as for
 * fp8bq_hyperball_step.
 *
 *   jobs[j]  w [R, C] FP32 (ldw >= C), read and written; g [R, C] of element type gt (ldg >= C);
 *            C % 8 == 0; radius >= 0 and finite (0: no projection); norms NULL or two 4-byte-aligned
 *            device floats (||g||, ||w|| after the update, before the projection).  A job with
 *            R == 0 or C == 0 is skipped (its pointers are not read).
 *   count    0 .. FP8BQ_MAX_HYPERBALL_JOBS (else FP8BQ_ERR_VALUE); 0 is a no-op.
 *   gt, lr, weight_decay, eps  shared by every job, as for fp8bq_hyperball_step.
 *   ws       at least fp8bq_hyperball_batch_workspace_size(count) bytes, 16-byte aligned (may be NULL
 *            when every job is empty).
 * The host array jobs is read during the call only.  Errors: as fp8bq_hyperball_step for any job
 * (the first failing job's status); FP8BQ_ERR_OVERLAP also when a job's w or norms overlaps another
 * job's w, g or norms, or any job's memory overlaps ws.  On an error nothing is enqueued.
 */
#define FP8BQ_MAX_HYPERBALL_JOBS 32
typedef struct {
  float* w;
  int64_t ldw;
  const void* g;
  int64_t ldg;
  int64_t R, C;
  double radius;
  float* norms;
} fp8bq_hyperball_job;
size_t fp8bq_hyperball_batch_workspace_size(int count);
int fp8bq_hyperball_step_batch(const fp8bq_hyperball_job* jobs, int count, fp8bq_in gt, double lr,
                               double weight_decay, double eps, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes the given GEMM needs at these sizes on the current device (0 if none).
 * Returns 0 for invalid arguments too; the GEMM call itself reports those. */
size_t fp8bq_gemm_workspace_size(fp8bq_op op, int64_t M, int64_t N, int64_t K);

/* The launch plan the given GEMM uses at these sizes on the current device: the output tile of
 * one work unit (*tile_m x *tile_n output rows x columns in the kernel's frame: fprop [M, N],
 * dgrad [M, K], wgrad [N, K]) and the number of parts the contraction is split into (*split_k;
 * 1 = no split, > 1 = FP32 partial sums in the workspace followed by a reduction pass).  The
 * plan is a deterministic function of (op, M, N, K) and the device's compute-unit count.
 * Returns FP8BQ_ERR_NULL if an output pointer is NULL, FP8BQ_ERR_SHAPE for an unknown op, a
 * negative size or a product too large for one launch (see FP8BQ_ERR_SHAPE); writes nothing then. */
int fp8bq_gemm_plan(fp8bq_op op, int64_t M, int64_t N, int64_t K, int32_t* tile_m, int32_t* tile_n,
                    int32_t* split_k);

/*
 * Streaming copy of `bytes` bytes from src to dst (device memory): the bandwidth reference that the
 * quantize passes are measured against.  It is not an operation of the layer: the pages define no
 * copy, and no other entry point uses it.  16-byte non-temporal loads and stores with a grid sized
 * from the device's compute units.
 *
 *   src, dst  16-byte aligned device pointers; the ranges [src, src+bytes) and [dst, dst+bytes)
 *             must not overlap.
 *   bytes     a multiple of 16, below 2^48; 0 is a no-op.
 *
 * Errors: FP8BQ_ERR_SHAPE (bytes not a multiple of 16, or too large), FP8BQ_ERR_NULL,
 * FP8BQ_ERR_ALIGN, FP8BQ_ERR_OVERLAP, FP8BQ_ERR_DEVICE, FP8BQ_ERR_LAUNCH.
 */
int fp8bq_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fp8bq_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int fp8bq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_H_ */
