// Streaming copy: the bandwidth reference the quantize passes are measured against (not part of the
// layer).  16-byte non-temporal loads and stores, four in flight per thread, a grid of 32 workgroups
// per compute unit striding over the buffer: the form that moved the most bytes per second among
// the plain copies tried on MI355X (6.0 TB/s read + write, against 5.5 TB/s with temporal accesses
// and 5.1 TB/s for the runtime's device-to-device copy).

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8bq {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4s* __restrict__ src, u32x4s* __restrict__ dst,
                                                          int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256 * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x; base < n; base += stride) {
    u32x4s v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, int cus, hipStream_t st) {
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t per_block = 256 * kCopyUnroll;
  int64_t blocks = (n + per_block - 1) / per_block;
  const int64_t cap = 32 * (int64_t)(cus > 0 ? cus : 256);
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const u32x4s*>(src), reinterpret_cast<u32x4s*>(dst), n);
  return hipGetLastError();
}

}  // namespace fp8bq
