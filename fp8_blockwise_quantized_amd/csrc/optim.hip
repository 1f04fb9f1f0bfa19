// Hyperball normalized weight update for gfx950, with the fixed-radius projection.
//
// The update ("用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析", section
// "Hyperball 优化：让 FP8 训练不爆炸", HyperballSGD.step): keep only the gradient's direction,
//   n = max(||g||_2, eps);   w <- w * (1 - lr * wd) - lr * g / n   (decoupled weight decay).
// The projection ("小团队也能预训练！普罗2B：RTX5090训练成本不到5090美元", MuonH paragraph; "Puro-2B:
// Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090", "方法关键点", MuonH bullet): after the
// update the weight goes back onto a fixed radius R, w <- R * w / ||w||_F (R = 0: none; a zero
// weight stays zero).  The gradient norm is also reported (the pages' debugging advice, section
// "调试 FP8 训练的关键步骤", is to watch it).
//
// Both passes are HBM-bound elementwise sweeps.  Global norms gate every element, so the step reads
// first and writes once:
//   1. per-block fp64 partial sums of g*g and, when the projection or the norms need them, of w*w
//      and w*g (reads g, and w);
//   2. the update, whose blocks each reduce those partials (fixed order: every block gets the same
//      values) to the step coefficient c = fp32(-lr / n) and, with d = fp32(1 - lr * wd), to the
//      updated weight's norm from the expansion ||w d + g c||^2 = d^2 sum w^2 + 2 d c sum wg +
//      c^2 sum g^2, then to the projection factor; it reads w and g and writes w once.
// That is 16 bytes per element (BF16 g) against 20 for a third sweep over the updated weight.  The
// expansion is evaluated in fp64 over exact fp64 products of fp32 values; it differs from the norm
// of the rounded FP32 weights by about 2^-24 relative, well inside the FP32 update's own error.
// Results are deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "optim.hpp"

namespace fp8bq {

namespace {

constexpr int kRowsPerIter = 4;

// 8 consecutive values as fp32 (FP32: two 16-byte loads; BF16: one).
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16lo(w.x); v[1] = bf16hi(w.x);
  v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
  v[4] = bf16lo(w.z); v[5] = bf16hi(w.z);
  v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Sum over the block (256 threads) in fp64; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Visit 8-element chunks: rows strided by the grid, kRowsPerIter rows per iteration so each thread
// keeps several loads in flight.
// (bid, nblk): this block's index among the nblk blocks that sweep the matrix.
template <typename F>
__device__ __forceinline__ void for_rows(int64_t R, int64_t C, uint32_t bid, uint32_t nblk, F&& f) {
  const int64_t chunks = C / 8;
  for (int64_t r0 = (int64_t)bid * kRowsPerIter; r0 < R; r0 += (int64_t)nblk * kRowsPerIter)
    for (int64_t c8 = threadIdx.x; c8 < chunks; c8 += blockDim.x) f(r0, 8 * c8);
}

// Pass 1: block bid's fp64 sums of g*g and, with WITH_W, of w*w and w*g, into partial[bid],
// partial[kHyperballBlocks + bid] and partial[2 * kHyperballBlocks + bid].
template <typename TG, bool WITH_W>
__device__ __forceinline__ void sums_body(const float* __restrict__ w, int64_t ldw, const TG* __restrict__ g,
                                          int64_t ldg, int64_t R, int64_t C, double* __restrict__ partial,
                                          uint32_t bid, uint32_t nblk, double* red) {
  double sgg = 0.0, sww = 0.0, swg = 0.0;
  for_rows(R, C, bid, nblk, [&](int64_t r0, int64_t c) {
    float gv[kRowsPerIter][8], wv[kRowsPerIter][8];
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
        load8(g + (r0 + i) * ldg + c, gv[i]);
        if constexpr (WITH_W) load8(w + (r0 + i) * ldw + c, wv[i]);
      }
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const double gd = gv[i][k];
          sgg = __builtin_fma(gd, gd, sgg);
          if constexpr (WITH_W) {
            const double wd = wv[i][k];
            sww = __builtin_fma(wd, wd, sww);
            swg = __builtin_fma(wd, gd, swg);
          }
        }
      }
  });
  double t = block_sum(sgg, red);
  if (threadIdx.x == 0) partial[bid] = t;
  if constexpr (WITH_W) {
    __syncthreads();
    t = block_sum(sww, red);
    if (threadIdx.x == 0) partial[kHyperballBlocks + bid] = t;
    __syncthreads();
    t = block_sum(swg, red);
    if (threadIdx.x == 0) partial[2 * kHyperballBlocks + bid] = t;
  }
}

template <typename TG, bool WITH_W>
__global__ __launch_bounds__(256) void hyperball_sums_kernel(const float* __restrict__ w, int64_t ldw,
                                                             const TG* __restrict__ g, int64_t ldg, int64_t R,
                                                             int64_t C, double* __restrict__ partial) {
  __shared__ double red[4];
  sums_body<TG, WITH_W>(w, ldw, g, ldg, R, C, partial, blockIdx.x, gridDim.x, red);
}

// Fixed-order sum of n partials by one block of 256 threads; every thread gets the result.
__device__ __forceinline__ double sum_partials(const double* partial, int n, double* red) {
  __shared__ double bc;
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s += partial[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) bc = s;
  __syncthreads();
  s = bc;
  __syncthreads();  // red and bc are reused
  return s;
}

// Pass 2: w <- fp32(fp32(w * d) + fp32(g * c)), times fp32(radius / ||w d + g c||) with PROJ.
// c = fp32(-lr / max(||g||, eps)), 0 for an all-zero gradient (whose move is zero whatever eps is).
// With WITH_W the updated weight's norm comes from the sums of pass 1; block 0 reports ||g|| and
// that norm if asked.
template <typename TG, bool WITH_W, bool PROJ>
__device__ __forceinline__ void update_body(float* __restrict__ w, int64_t ldw, const TG* __restrict__ g, int64_t ldg,
                                            int64_t R, int64_t C, float d, const double* __restrict__ partial,
                                            double lr, double eps, double radius, float* __restrict__ norms,
                                            uint32_t bid, uint32_t nblk, double* red) {
  const int np = (int)nblk;
  const double sgg = sum_partials(partial, np, red);
  const double gn = __builtin_sqrt(sgg);
  const double n = gn > eps ? gn : eps;
  const float c = gn > 0.0 ? (float)(-lr / n) : 0.0f;
  float f = 1.0f;
  if constexpr (WITH_W) {
    const double sww = sum_partials(partial + kHyperballBlocks, np, red);
    const double swg = sum_partials(partial + 2 * kHyperballBlocks, np, red);
    const double dd = d, cd = c;
    double wn2 = dd * dd * sww + 2.0 * dd * cd * swg + cd * cd * sgg;
    wn2 = wn2 > 0.0 ? wn2 : 0.0;  // (rounding can only push an exactly zero weight below zero)
    const double wn = __builtin_sqrt(wn2);
    if (PROJ && wn > 0.0) f = (float)(radius / wn);
    if (norms && bid == 0 && threadIdx.x == 0) norms[1] = (float)wn;
  }
  if (norms && bid == 0 && threadIdx.x == 0) norms[0] = (float)gn;
  for_rows(R, C, bid, nblk, [&](int64_t r0, int64_t col) {
    float wv[kRowsPerIter][8], gv[kRowsPerIter][8];
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
        load8(w + (r0 + i) * ldw + col, wv[i]);
        load8(g + (r0 + i) * ldg + col, gv[i]);
      }
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          wv[i][k] = __fadd_rn(__fmul_rn(wv[i][k], d), __fmul_rn(gv[i][k], c));
          if constexpr (PROJ) wv[i][k] = __fmul_rn(wv[i][k], f);
        }
        store8(w + (r0 + i) * ldw + col, wv[i]);
      }
  });
}

template <typename TG, bool WITH_W, bool PROJ>
__global__ __launch_bounds__(256) void hyperball_update_kernel(float* __restrict__ w, int64_t ldw,
                                                               const TG* __restrict__ g, int64_t ldg, int64_t R,
                                                               int64_t C, float d, const double* __restrict__ partial,
                                                               double lr, double eps, double radius,
                                                               float* __restrict__ norms) {
  __shared__ double red[4];
  update_body<TG, WITH_W, PROJ>(w, ldw, g, ldg, R, C, d, partial, lr, eps, radius, norms, blockIdx.x, gridDim.x, red);
}

// Several matrices per launch: the blocks of job j are start[j] .. start[j+1]-1, hyperball_blocks(R)
// of them as a single call would launch, each with that call's block index, so every job gets the
// single call's partial sums, reduction order and results, bit for bit.  A job uses the projection
// when its radius is positive and the w sums when it has a radius or reports norms, as a single
// call does; the job search is a scalar scan over at most kMaxHyperballJobs prefix sums.
__device__ __forceinline__ int batch_job(const HyperballBatch& b, uint32_t blk) {
  int j = 0;
  while (j + 1 < b.count && blk >= b.start[j + 1]) ++j;
  return __builtin_amdgcn_readfirstlane(j);
}

template <typename TG>
__global__ __launch_bounds__(256) void hyperball_sums_batch_kernel(HyperballBatch b) {
  __shared__ double red[4];
  const int j = batch_job(b, blockIdx.x);
  const uint32_t bid = blockIdx.x - b.start[j], nblk = b.start[j + 1] - b.start[j];
  double* partial = b.partial + (size_t)j * 3 * kHyperballBlocks;
  const TG* g = (const TG*)b.g[j];
  if (b.radius[j] > 0.0 || b.norms[j] != nullptr)
    sums_body<TG, true>(b.w[j], b.ldw[j], g, b.ldg[j], b.R[j], b.C[j], partial, bid, nblk, red);
  else
    sums_body<TG, false>(b.w[j], b.ldw[j], g, b.ldg[j], b.R[j], b.C[j], partial, bid, nblk, red);
}

template <typename TG>
__global__ __launch_bounds__(256) void hyperball_update_batch_kernel(HyperballBatch b, float d, double lr,
                                                                     double eps) {
  __shared__ double red[4];
  const int j = batch_job(b, blockIdx.x);
  const uint32_t bid = blockIdx.x - b.start[j], nblk = b.start[j + 1] - b.start[j];
  const double* partial = b.partial + (size_t)j * 3 * kHyperballBlocks;
  const TG* g = (const TG*)b.g[j];
  if (b.radius[j] > 0.0)
    update_body<TG, true, true>(b.w[j], b.ldw[j], g, b.ldg[j], b.R[j], b.C[j], d, partial, lr, eps, b.radius[j],
                                b.norms[j], bid, nblk, red);
  else if (b.norms[j] != nullptr)
    update_body<TG, true, false>(b.w[j], b.ldw[j], g, b.ldg[j], b.R[j], b.C[j], d, partial, lr, eps, 0.0,
                                 b.norms[j], bid, nblk, red);
  else
    update_body<TG, false, false>(b.w[j], b.ldw[j], g, b.ldg[j], b.R[j], b.C[j], d, partial, lr, eps, 0.0,
                                  nullptr, bid, nblk, red);
}

template <typename TG, bool WITH_W, bool PROJ>
hipError_t launch_pair(float* w, int64_t ldw, const TG* g, int64_t ldg, int64_t R, int64_t C, float d, double lr,
                       double eps, double radius, float* norms, double* partial, int nb, hipStream_t st) {
  hipLaunchKernelGGL((hyperball_sums_kernel<TG, WITH_W>), dim3(nb), dim3(256), 0, st, (const float*)w, ldw, g, ldg, R,
                     C, partial);
  const hipError_t e = hipGetLastError();  // a failed launch stops the call before the update
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hyperball_update_kernel<TG, WITH_W, PROJ>), dim3(nb), dim3(256), 0, st, w, ldw, g, ldg, R, C, d,
                     (const double*)partial, lr, eps, radius, norms);
  return hipGetLastError();
}

template <typename TG>
hipError_t launch_batch_t(const HyperballBatch& b, float d, double lr, double eps, hipStream_t st) {
  const unsigned grid = b.start[b.count];
  hipLaunchKernelGGL((hyperball_sums_batch_kernel<TG>), dim3(grid), dim3(256), 0, st, b);
  const hipError_t e = hipGetLastError();  // a failed launch stops the call before the update
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((hyperball_update_batch_kernel<TG>), dim3(grid), dim3(256), 0, st, b, d, lr, eps);
  return hipGetLastError();
}

template <typename TG>
hipError_t launch_t(float* w, int64_t ldw, const void* g, int64_t ldg, int64_t R, int64_t C, double lr, double wd,
                    double eps, double radius, float* norms, void* ws, hipStream_t st) {
  const int nb = hyperball_blocks(R);
  double* partial = reinterpret_cast<double*>(ws);
  const float d = (float)(1.0 - lr * wd);
  const TG* gt = (const TG*)g;
  if (radius > 0.0) return launch_pair<TG, true, true>(w, ldw, gt, ldg, R, C, d, lr, eps, radius, norms, partial, nb, st);
  if (norms) return launch_pair<TG, true, false>(w, ldw, gt, ldg, R, C, d, lr, eps, radius, norms, partial, nb, st);
  return launch_pair<TG, false, false>(w, ldw, gt, ldg, R, C, d, lr, eps, radius, norms, partial, nb, st);
}

}  // namespace

int hyperball_blocks(int64_t R) {
  const int64_t want = (R + kRowsPerIter - 1) / kRowsPerIter;
  return (int)(want < kHyperballBlocks ? (want > 0 ? want : 1) : kHyperballBlocks);
}

hipError_t launch_hyperball_step(float* w, int64_t ldw, const void* g, int gt, int64_t ldg, int64_t R, int64_t C,
                                 double lr, double wd, double eps, double radius, float* norms, void* ws,
                                 hipStream_t st) {
  if (gt == 0) return launch_t<uint16_t>(w, ldw, g, ldg, R, C, lr, wd, eps, radius, norms, ws, st);
  return launch_t<float>(w, ldw, g, ldg, R, C, lr, wd, eps, radius, norms, ws, st);
}

hipError_t launch_hyperball_batch(const HyperballBatch& b, int gt, double lr, double wd, double eps, hipStream_t st) {
  const float d = (float)(1.0 - lr * wd);
  if (gt == 0) return launch_batch_t<uint16_t>(b, d, lr, eps, st);
  return launch_batch_t<float>(b, d, lr, eps, st);
}

}  // namespace fp8bq
