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
// All passes are HBM-bound elementwise sweeps.  A global norm is needed before any element can be
// updated, so the step is: partial sums of squares of g (fp64, per block) -> the update, whose
// blocks each first reduce those partials to the step coefficient and which also sums the squares
// of the new weights -> (with a radius) the scaling pass, whose blocks each reduce those to the
// projection factor.  Every block combines the partials in the same fixed order, so all blocks use
// the same coefficient and results are deterministic.
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
template <typename F>
__device__ __forceinline__ void for_rows(int64_t R, int64_t C, F&& f) {
  const int64_t chunks = C / 8;
  for (int64_t r0 = (int64_t)blockIdx.x * kRowsPerIter; r0 < R; r0 += (int64_t)gridDim.x * kRowsPerIter)
    for (int64_t c8 = threadIdx.x; c8 < chunks; c8 += blockDim.x) f(r0, 8 * c8);
}

template <typename TG>
__global__ __launch_bounds__(256) void sumsq_kernel(const TG* __restrict__ g, int64_t R, int64_t C, int64_t ldg,
                                                    double* __restrict__ partial) {
  __shared__ double red[4];
  double s = 0.0;
  for_rows(R, C, [&](int64_t r0, int64_t c) {
    float v[kRowsPerIter][8];
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) load8(g + (r0 + i) * ldg + c, v[i]);
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s = __builtin_fma((double)v[i][k], (double)v[i][k], s);
      }
  });
  const double t = block_sum(s, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

// Fixed-order sum of n partials by one block of 256 threads.
__device__ __forceinline__ double sum_partials(const double* partial, int n, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s += partial[i];
  return block_sum(s, red);
}

// coef = fp32(-lr / max(||g||, eps)) (0 for an all-zero gradient, whose move is zero whatever eps
// is), from the gradient's partial sums; block 0 reports ||g|| if asked.
__device__ __forceinline__ float grad_coef(const double* partial, int n, double lr, double eps, float* norms,
                                           double* red) {
  __shared__ double bc;
  const double s = sum_partials(partial, n, red);
  if (threadIdx.x == 0) {
    bc = s;
    if (norms && blockIdx.x == 0) norms[0] = (float)__builtin_sqrt(s);
  }
  __syncthreads();
  const double gn = __builtin_sqrt(bc);
  const double d = gn > eps ? gn : eps;
  __syncthreads();  // red is reused by the caller
  return gn > 0.0 ? (float)(-lr / d) : 0.0f;
}

// w <- w * decay + g * coef (three fp32 roundings); with PROJ also the block's sum of squares of
// the new weights.
template <typename TG, bool PROJ>
__global__ __launch_bounds__(256) void hyperball_update_kernel(float* __restrict__ w, int64_t ldw,
                                                               const TG* __restrict__ g, int64_t ldg, int64_t R,
                                                               int64_t C, float decay, const double* __restrict__ pg,
                                                               int npg, double lr, double eps,
                                                               float* __restrict__ norms,
                                                               double* __restrict__ partial) {
  __shared__ double red[4];
  const float coef = grad_coef(pg, npg, lr, eps, norms, red);
  double s = 0.0;
  for_rows(R, C, [&](int64_t r0, int64_t c) {
    float wv[kRowsPerIter][8], gv[kRowsPerIter][8];
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
        load8(w + (r0 + i) * ldw + c, wv[i]);
        load8(g + (r0 + i) * ldg + c, gv[i]);
      }
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          wv[i][k] = __fadd_rn(__fmul_rn(wv[i][k], decay), __fmul_rn(gv[i][k], coef));
          if constexpr (PROJ) s = __builtin_fma((double)wv[i][k], (double)wv[i][k], s);
        }
        store8(w + (r0 + i) * ldw + c, wv[i]);
      }
  });
  if constexpr (PROJ) {
    const double t = block_sum(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = t;
  }
}

// ||w|| after the update, from its partial sums (the same value in every block); block 0 reports it
// if asked.
__device__ __forceinline__ double weight_norm(const double* partial, int n, float* norms, double* red) {
  __shared__ double bc;
  const double s = sum_partials(partial, n, red);
  if (threadIdx.x == 0) {
    bc = s;
    if (norms && blockIdx.x == 0) norms[1] = (float)__builtin_sqrt(s);
  }
  __syncthreads();
  return __builtin_sqrt(bc);
}

// Only the norm, for a step without a projection that reports it.
__global__ __launch_bounds__(256) void weight_norm_kernel(const double* __restrict__ partial, int n,
                                                          float* __restrict__ norms) {
  __shared__ double red[4];
  weight_norm(partial, n, norms, red);
}

// w <- w * fp32(radius / ||w||) (a zero weight is left as it is).
__global__ __launch_bounds__(256) void scale_kernel(float* __restrict__ w, int64_t ldw, int64_t R, int64_t C,
                                                    const double* __restrict__ pw, int npw, double radius,
                                                    float* __restrict__ norms) {
  __shared__ double red[4];
  const double wn = weight_norm(pw, npw, norms, red);
  const float f = wn > 0.0 ? (float)(radius / wn) : 1.0f;
  for_rows(R, C, [&](int64_t r0, int64_t c) {
    float wv[kRowsPerIter][8];
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) load8(w + (r0 + i) * ldw + c, wv[i]);
#pragma unroll
    for (int i = 0; i < kRowsPerIter; ++i)
      if (r0 + i < R) {
#pragma unroll
        for (int k = 0; k < 8; ++k) wv[i][k] = __fmul_rn(wv[i][k], f);
        store8(w + (r0 + i) * ldw + c, wv[i]);
      }
  });
}

template <typename TG>
hipError_t launch_t(float* w, int64_t ldw, const void* g, int64_t ldg, int64_t R, int64_t C, double lr, double wd,
                    double eps, double radius, float* norms, void* ws, hipStream_t st) {
  const int nb = hyperball_blocks(R);
  double* pg = reinterpret_cast<double*>(ws);
  double* pw = pg + kHyperballBlocks;
  const float decay = (float)(1.0 - lr * wd);
  hipLaunchKernelGGL((sumsq_kernel<TG>), dim3(nb), dim3(256), 0, st, (const TG*)g, R, C, ldg, pg);
  if (radius > 0.0 || norms) {
    hipLaunchKernelGGL((hyperball_update_kernel<TG, true>), dim3(nb), dim3(256), 0, st, w, ldw, (const TG*)g, ldg, R,
                       C, decay, (const double*)pg, nb, lr, eps, norms, pw);
    if (radius > 0.0)
      hipLaunchKernelGGL(scale_kernel, dim3(nb), dim3(256), 0, st, w, ldw, R, C, (const double*)pw, nb, radius,
                         norms);
    else
      hipLaunchKernelGGL(weight_norm_kernel, dim3(1), dim3(256), 0, st, (const double*)pw, nb, norms);
  } else {
    hipLaunchKernelGGL((hyperball_update_kernel<TG, false>), dim3(nb), dim3(256), 0, st, w, ldw, (const TG*)g, ldg,
                       R, C, decay, (const double*)pg, nb, lr, eps, norms, pw);
  }
  return hipGetLastError();
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

}  // namespace fp8bq
