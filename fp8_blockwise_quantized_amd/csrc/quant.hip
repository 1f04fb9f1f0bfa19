// FP8 quantize kernels for gfx950: blockwise 1x128 (activations), 128x1 (token axis, transposed
// output for wgrad), both at once (dual), 128x128 (weights, optionally also transposed, one weight or
// several per launch), and the per-tensor delayed-scaling variant at the end of the file.
//
// Rule per group ("用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析", section
// "核心挑战：Scale Factor 管理", FP8Linear._quantize): amax = max|x|; s = max(RN(amax/fmt_max), 1e-12);
// q = RNE code of clamp(RN(x/s), +-fmt_max).  Group shapes: activations 1-D groups of 128, weights
// 128x128 tiles ("Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090", "方法关键点",
// bullet "FP8 blockwise 混合精度").
//
// The blockwise passes are HBM-bound (about 3 bytes moved per element from BF16).  Each reads its input
// once with 16-byte coalesced loads, keeps the group in registers, reduces amax with DPP row
// rotations (1x128, 128x128) or through LDS (128x1, whose groups run down columns), and writes codes
// with 8- or 16-byte stores.  The division x/s uses the exact reciprocal-and-residual form in
// div_by_scale (3 VALU ops instead of an IEEE divide sequence), which returns the IEEE quotient bit
// for bit wherever it can change a code.  The blockwise passes skip the clamp, which changes no code
// there (blockwise_quotient), and compute each group scale once per group rather than in every lane
// that holds part of the group (row16_max_scatter).

#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8bq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Plain (temporal) global accesses: inputs are often read again (an activation feeds both the 1x128
// and the 128x1 pass) and codes are read next by the GEMM, so letting them stay in the 256 MB
// Infinity Cache pays; non-temporal hints measured faster only on tensors larger than that cache.
__device__ __forceinline__ void store_codes8(uint8_t* p, uint2 w) {
  *reinterpret_cast<u32x2*>(p) = (u32x2){w.x, w.y};
}
__device__ __forceinline__ void store_codes16(uint8_t* p, uint4 w) {
  *reinterpret_cast<u32x4*>(p) = (u32x4){w.x, w.y, w.z, w.w};
}

// Load 8 consecutive input elements (16 bytes of BF16 or 32 bytes of FP32) as fp32.
template <typename TIn>
struct Load8;
template <>
struct Load8<uint16_t> {
  static __device__ __forceinline__ void run(const uint16_t* p, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x);
    v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
    v[4] = bf16lo(w.z); v[5] = bf16hi(w.z);
    v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
  }
};
template <>
struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *(reinterpret_cast<const f32x4*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Quantize 8 values with the group's (s, r) into two dwords of codes.  CLAMP: clamp the quotients to
// +-fmt_max before converting, which a per-tensor scale from a running amax needs (the tensor can
// exceed it); a blockwise scale comes from the group's own amax, so the quotients need no clamp
// (blockwise_quotient).
template <int FMT, bool CLAMP = false>
__device__ __forceinline__ uint2 quant8(const float (&v)[8], float s, float r) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = CLAMP ? clamp_fmt<FMT>(div_by_scale(v[i], s, r)) : blockwise_quotient(v[i], s, r);
  return make_uint2(pack4<FMT>(y[0], y[1], y[2], y[3]), pack4<FMT>(y[4], y[5], y[6], y[7]));
}

// ---------------------------------------------------------------------------------------------
// 1x128: grid (ceil(R/64), C/128).  A block owns one 128-column group for 64 rows.  16 lanes (one
// DPP row) hold one group, 8 elements each; the 256 threads cover 16 rows per pass, 4 passes.
// ---------------------------------------------------------------------------------------------
constexpr int kQ1Rows = 64;

template <typename TIn, int FMT>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const TIn* __restrict__ x, int64_t R, int64_t ldx,
                                                          uint8_t* __restrict__ q, int64_t ldq,
                                                          float* __restrict__ s, int64_t lds) {
  const int t = threadIdx.x;
  const int l16 = t & 15;
  const int rsub = t >> 4;
  const int64_t g = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * kQ1Rows;
  const int64_t col = g * kGroup + 8 * l16;

  float v[4][8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t r = r0 + rsub + 16 * p;
    if (r < R) {
      Load8<TIn>::run(x + r * ldx + col, v[p]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.0f;
    }
  }
  // Each lane ends with one row's group amax (row l16 / 4) and computes that row's scale; the 16
  // lanes then take the four rows' scales from lanes 0, 4, 8, 12.
  float m[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    m[p] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m[p] = __builtin_fmaxf(m[p], __builtin_fabsf(v[p][i]));
  }
  const float sc_own = group_scale<FMT>(row16_max_scatter<4>(m, l16));
  const float rc_own = 1.0f / sc_own;
  const int own = l16 >> scatter_shift<4>();
  if ((l16 & 3) == 0 && r0 + rsub + 16 * own < R) s[g * lds + r0 + rsub + 16 * own] = sc_own;
  static_for<4>([&](auto P) {
    constexpr int p = decltype(P)::value;
    const float sc = row16_bcast<(p << scatter_shift<4>())>(sc_own);
    const float rc = row16_bcast<(p << scatter_shift<4>())>(rc_own);
    const int64_t r = r0 + rsub + 16 * p;
    if (r < R) store_codes8(q + r * ldq + col, quant8<FMT>(v[p], sc, rc));
  });
}

// ---------------------------------------------------------------------------------------------
// 128x1: grid (ceil(C/128), R/128).  A block owns rows 128*rb .. +127 and 128 columns (256-byte row
// segments of BF16).  Thread t holds an 8-row x 8-column patch (rows 8*(t>>4)+0..7, columns
// 8*(t&15)+0..7), i.e. 8 independent 16-byte loads.  Column amax goes through LDS; each column's
// 8 codes are packed into two dwords, staged transposed in LDS, and written as 16-byte runs along
// the token axis (128 contiguous bytes per column).
// ---------------------------------------------------------------------------------------------
constexpr int kQtCols = 128;

// LDS layouts of the 128-column tile kernels, chosen so that no access conflicts on LDS banks
// (64 banks of 4 bytes; a thread's 8 columns are 8*cc .. 8*cc+7, cc = t % 16, and the 4 row groups
// of a wave share them):
// - per-column arrays (partial maxima, scales) put column c at c + 4*(c/64): columns c and c+64,
//   which one instruction's lanes cc and cc+8 touch together, fall on different banks;
// - the transposed codes: column c's 128 codes (one byte per row) at byte 128*c + 128*(c/64), its
//   8-byte unit u (rows 8u .. 8u+7) at unit u ^ 2*((c ^ c/8) % 8).  The XOR value is even, so the
//   16-byte read of units 2h, 2h+1 stays one aligned access.
constexpr int kColPos = kQtCols + 4;   // entries per padded per-column array
constexpr int kRedStride = kColPos + 1;  // partial-maxima row stride (133: row groups 4 banks apart)
constexpr int kQtBytes = kQtCols * 128 + 128;
__device__ __forceinline__ int col_pos(int c) { return c + ((c >> 6) << 2); }
__device__ __forceinline__ int qt_off(int c, int u) {
  return (c << 7) + ((c >> 6) << 7) + ((u ^ (((c ^ (c >> 3)) & 7) << 1)) << 3);
}

template <typename TIn, int FMT>
__global__ __launch_bounds__(256) void quant_128x1_kernel(const TIn* __restrict__ x, int64_t C, int64_t ldx,
                                                          uint8_t* __restrict__ qt, int64_t ldqt,
                                                          float* __restrict__ st, int64_t ldst, uint32_t ncg) {
  __shared__ float red[16][kRedStride];
  __shared__ __attribute__((aligned(16))) float ssc[kColPos];
  __shared__ __attribute__((aligned(16))) float src[kColPos];
  __shared__ __attribute__((aligned(16))) uint8_t tileT[kQtBytes];

  const int t = threadIdx.x;
  const int cc = t & 15;
  const int rg = t >> 4;
  const TileRC tile = tile_of_block(ncg);
  const int64_t rb = tile.row;
  const int64_t c0 = tile.col * kQtCols;
  const int64_t col = c0 + 8 * cc;
  const bool cvalid = col < C;  // C % 8 == 0, so a chunk is all in or all out

  float v[8][8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int64_t r = rb * kGroup + 8 * rg + p;
    if (cvalid) {
      Load8<TIn>::run(x + r * ldx + col, v[p]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = __builtin_fabsf(v[0][i]);
#pragma unroll
    for (int p = 1; p < 8; ++p) m = __builtin_fmaxf(m, __builtin_fabsf(v[p][i]));
    red[rg][col_pos(8 * cc + i)] = m;
  }
  __syncthreads();
  if (t < kQtCols) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) m = __builtin_fmaxf(m, red[k][col_pos(t)]);
    const float sc = group_scale<FMT>(m);
    ssc[col_pos(t)] = sc;
    src[col_pos(t)] = 1.0f / sc;
    if (c0 + t < C) st[rb * ldst + c0 + t] = sc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 8 * cc + i;
    const float sc = ssc[col_pos(c)], rc = src[col_pos(c)];
    float y[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) y[p] = blockwise_quotient(v[p][i], sc, rc);
    const uint2 w = make_uint2(pack4<FMT>(y[0], y[1], y[2], y[3]), pack4<FMT>(y[4], y[5], y[6], y[7]));
    *reinterpret_cast<uint2*>(tileT + qt_off(c, rg)) = w;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int c = (t >> 3) + 32 * pass;
    const int ch = t & 7;
    if (c0 + c < C) {
      const uint4 codes = *reinterpret_cast<const uint4*>(tileT + qt_off(c, 2 * ch));
      store_codes16(qt + (c0 + c) * ldqt + rb * kGroup + 16 * ch, codes);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Both activation layouts from one read: grid (C/128, R/128), the 128x1 kernel's 128x128 tiles and
// thread mapping.  The 16 threads that share a row patch are one DPP row, so each of a thread's 8
// rows also gets its 1x128 group amax by DPP, and its 8 codes of that row go out as one 8-byte store
// (16 threads write the row's 128 contiguous bytes).  Codes and scales are those of the two separate
// kernels, bit for bit (same scale, division and conversion code).
// ---------------------------------------------------------------------------------------------
template <typename TIn, int FR, int FC>
__global__ __launch_bounds__(256) void quant_dual_kernel(const TIn* __restrict__ x, int64_t ldx,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ s, int64_t lds,
                                                         uint8_t* __restrict__ qt, int64_t ldqt,
                                                         float* __restrict__ st, int64_t ldst, uint32_t ncg) {
  __shared__ float red[16][kRedStride];
  __shared__ __attribute__((aligned(16))) float ssc[kColPos];
  __shared__ __attribute__((aligned(16))) float src[kColPos];
  __shared__ __attribute__((aligned(16))) uint8_t tileT[kQtBytes];

  const int t = threadIdx.x;
  const int cc = t & 15;
  const int rg = t >> 4;
  const TileRC tile = tile_of_block(ncg);
  const int64_t rb = tile.row;
  const int64_t g = tile.col;  // 128-column group
  const int64_t c0 = g * kQtCols;
  const int64_t col = c0 + 8 * cc;

  float v[8][8];
#pragma unroll
  for (int p = 0; p < 8; ++p) Load8<TIn>::run(x + (rb * kGroup + 8 * rg + p) * ldx + col, v[p]);

  // 1x128 groups: row r = 128*rb + 8*rg + p, columns c0 .. c0+127.  Each lane ends with one row's
  // group amax (row cc / 2) and computes that row's scale; the 16 lanes then take the eight rows'
  // scales from the even lanes.
  {
    float m[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      m[p] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m[p] = __builtin_fmaxf(m[p], __builtin_fabsf(v[p][i]));
    }
    const float sc_own = group_scale<FR>(row16_max_scatter<8>(m, cc));
    const float rc_own = 1.0f / sc_own;
    if ((cc & 1) == 0) s[g * lds + rb * kGroup + 8 * rg + (cc >> scatter_shift<8>())] = sc_own;
    static_for<8>([&](auto P) {
      constexpr int p = decltype(P)::value;
      const float sc = row16_bcast<(p << scatter_shift<8>())>(sc_own);
      const float rc = row16_bcast<(p << scatter_shift<8>())>(rc_own);
      store_codes8(q + (rb * kGroup + 8 * rg + p) * ldq + col, quant8<FR>(v[p], sc, rc));
    });
  }

  // 128x1 groups: column c0 + c, rows 128*rb .. +127 (as quant_128x1_kernel)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = __builtin_fabsf(v[0][i]);
#pragma unroll
    for (int p = 1; p < 8; ++p) m = __builtin_fmaxf(m, __builtin_fabsf(v[p][i]));
    red[rg][col_pos(8 * cc + i)] = m;
  }
  __syncthreads();
  if (t < kQtCols) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) m = __builtin_fmaxf(m, red[k][col_pos(t)]);
    const float sc = group_scale<FC>(m);
    ssc[col_pos(t)] = sc;
    src[col_pos(t)] = 1.0f / sc;
    st[rb * ldst + c0 + t] = sc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 8 * cc + i;
    const float sc = ssc[col_pos(c)], rc = src[col_pos(c)];
    float y[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) y[p] = blockwise_quotient(v[p][i], sc, rc);
    const uint2 w = make_uint2(pack4<FC>(y[0], y[1], y[2], y[3]), pack4<FC>(y[4], y[5], y[6], y[7]));
    *reinterpret_cast<uint2*>(tileT + qt_off(c, rg)) = w;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int c = (t >> 3) + 32 * pass;
    const int ch = t & 7;
    const uint4 codes = *reinterpret_cast<const uint4*>(tileT + qt_off(c, 2 * ch));
    store_codes16(qt + (c0 + c) * ldqt + rb * kGroup + 16 * ch, codes);
  }
}

// ---------------------------------------------------------------------------------------------
// 128x128: grid (K/128, N/128), one block per weight tile.  Thread t holds rows (t>>4) + 16*p,
// p = 0..7, columns 8*(t&15)+0..7 (64 values).  amax: DPP within rows of 16 lanes, readlane across
// the wave, LDS across the 4 waves.
// ---------------------------------------------------------------------------------------------
template <typename TIn, int FMT>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const TIn* __restrict__ w, int64_t ldw,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ s, int64_t lds, uint32_t nkb) {
  __shared__ float wmax[4];
  const int t = threadIdx.x;
  const int l16 = t & 15;
  const int rsub = t >> 4;
  const TileRC tile = tile_of_block(nkb);
  const int64_t kb = tile.col, nb = tile.row;
  const int64_t col = kb * kGroup + 8 * l16;

  float v[8][8];
#pragma unroll
  for (int p = 0; p < 8; ++p) Load8<TIn>::run(w + (nb * kGroup + rsub + 16 * p) * ldw + col, v[p]);
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[p][i]));
  m = wave_max(m);
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  const float amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
  const float sc = group_scale<FMT>(amax);
  const float rc = 1.0f / sc;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    store_codes8(q + (nb * kGroup + rsub + 16 * p) * ldq + col, quant8<FMT>(v[p], sc, rc));
  }
  if (t == 0) s[nb * lds + kb] = sc;
}

// Per-tensor scale of the delayed-scaling rule (below), computed by every block of the code pass
// from the amax pass's partial maxima and the running amax it saved: cur = max of the partials;
// fresh = fp32(cur * b2), rounded to BF16 when the tensor is BF16 (the listing weights the current
// amax in the tensor's own type); a = fp32(fp32(a_old * b1) + fresh); s = max(fp32(a / fmt_max),
// 1e-12).  The first block stores the new running amax and the scale.  b1 = fp32(beta),
// b2 = fp32(1 - beta).
struct TensorScaleArgs {
  const float* partial;  // n partial maxima, then the running amax as it was before this call
  int n;
  float b1, b2;
  float* amax;
  float* s;
};

template <typename TIn, int FMT>
__device__ __forceinline__ float tensor_scale(const TensorScaleArgs& a) {
  __shared__ float tmax[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) m = __builtin_fmaxf(m, a.partial[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) tmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float cur = __builtin_fmaxf(__builtin_fmaxf(tmax[0], tmax[1]), __builtin_fmaxf(tmax[2], tmax[3]));
  float fresh = __fmul_rn(cur, a.b2);
  if constexpr (sizeof(TIn) == 2) fresh = round_bf16(fresh);
  const float am = __fadd_rn(__fmul_rn(a.partial[kTensorAmaxBlocks], a.b1), fresh);
  const float sc = group_scale<FMT>(am);
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    a.amax[0] = am;
    a.s[0] = sc;
  }
  return sc;
}

// ---------------------------------------------------------------------------------------------
// 128x128 with a transposed copy: grid (K/128, N/128), one block per weight tile, the 128x1
// kernel's thread mapping (8 consecutive rows x 8 columns per thread).  The tile's amax goes
// through readlane and LDS; codes are written row-major (8-byte runs) and, staged transposed in
// LDS, as W^T codes (16-byte runs), the operand layout of dgrad's contraction over N.
// TENSOR: the per-tensor scale comes from tensor_scale (the delayed-scaling rule below; s and lds
// are unused) and the codes are those of the input's BF16 copy.
// ---------------------------------------------------------------------------------------------
template <typename TIn, int FMT, bool TENSOR>
__device__ __forceinline__ void weight_dual_tile(const TIn* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q,
                                                 int64_t ldq, float* __restrict__ s, int64_t lds,
                                                 uint8_t* __restrict__ qt, int64_t ldqt, const TensorScaleArgs& ta,
                                                 int64_t nb, int64_t kb) {
  __shared__ float wmax[4];
  __shared__ __attribute__((aligned(16))) uint8_t tileT[kQtBytes];
  const int t = threadIdx.x;
  const int cc = t & 15;
  const int rg = t >> 4;
  const int64_t col = kb * kGroup + 8 * cc;

  float v[8][8];
#pragma unroll
  for (int p = 0; p < 8; ++p) Load8<TIn>::run(w + (nb * kGroup + 8 * rg + p) * ldw + col, v[p]);
  float sc;
  if constexpr (TENSOR) {
    sc = tensor_scale<TIn, FMT>(ta);
    if constexpr (sizeof(TIn) == 4) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][i] = round_bf16(v[p][i]);
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[p][i]));
    m = wave_max(m);
    if ((t & 63) == 0) wmax[t >> 6] = m;
    __syncthreads();
    const float amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    sc = group_scale<FMT>(amax);
  }
  const float rc = 1.0f / sc;
  uint8_t cb[8][8];  // codes [row p][column i]
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint2 wd = quant8<FMT, TENSOR>(v[p], sc, rc);
    store_codes8(q + (nb * kGroup + 8 * rg + p) * ldq + col, wd);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cb[p][i] = (uint8_t)(wd.x >> (8 * i));
      cb[p][4 + i] = (uint8_t)(wd.y >> (8 * i));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      lo |= (uint32_t)cb[p][i] << (8 * p);
      hi |= (uint32_t)cb[4 + p][i] << (8 * p);
    }
    *reinterpret_cast<uint2*>(tileT + qt_off(8 * cc + i, rg)) = make_uint2(lo, hi);
  }
  if (!TENSOR && t == 0) s[nb * lds + kb] = sc;
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int c = (t >> 3) + 32 * pass;
    const int ch = t & 7;
    const uint4 codes = *reinterpret_cast<const uint4*>(tileT + qt_off(c, 2 * ch));
    store_codes16(qt + (kb * kGroup + c) * ldqt + nb * kGroup + 16 * ch, codes);
  }
}

template <typename TIn, int FMT, bool TENSOR = false>
__global__ __launch_bounds__(256) void quant_128x128_dual_kernel(const TIn* __restrict__ w, int64_t ldw,
                                                                 uint8_t* __restrict__ q, int64_t ldq,
                                                                 float* __restrict__ s, int64_t lds,
                                                                 uint8_t* __restrict__ qt, int64_t ldqt,
                                                                 TensorScaleArgs ta, uint32_t nkb) {
  const TileRC tile = tile_of_block(nkb);
  weight_dual_tile<TIn, FMT, TENSOR>(w, ldw, q, ldq, s, lds, qt, ldqt, ta, tile.row, tile.col);
}

// Several weights in one launch: the tiles of job j are blocks start[j] .. start[j+1]-1, each job's
// tiles in the single-weight kernel's order, so every job gets exactly that kernel's codes and scales.
// The host lists only jobs with tiles (start strictly increasing); the job search is a scalar scan.
template <typename TIn, int FMT>
__global__ __launch_bounds__(256) void quant_weights_dual_kernel(WeightDualBatch b) {
  const uint32_t blk = blockIdx.x;
  int j = 0;
  while (j + 1 < b.count && blk >= b.start[j + 1]) ++j;
  const uint32_t local = blk - b.start[j];
  const uint32_t nkb = b.nkb[j];
  const uint32_t r = __builtin_amdgcn_readfirstlane(local / nkb);
  weight_dual_tile<TIn, FMT, false>(reinterpret_cast<const TIn*>(b.w[j]), b.ldw[j], b.q[j], b.ldq[j], b.s[j],
                                    b.lds[j], b.qt[j], b.ldqt[j], TensorScaleArgs{}, (int64_t)r,
                                    (int64_t)(local - r * nkb));
}

// ---------------------------------------------------------------------------------------------
// Per-tensor delayed scaling ("用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析",
// section "核心挑战：Scale Factor 管理", FP8Linear: _update_amax, _quantize, forward).  One scale per
// tensor from a running amax: the tensor's current max|x| (of the values as given) updates the
// running value, a = fp32(fp32(a * beta) + fresh) with fresh = cur * (1 - beta) in the tensor's
// type (fp32, or fp32 rounded to BF16 for a BF16 tensor), and the tensor's BF16 copy is quantized
// with s = max(fp32(a / fmt_max), 1e-12).  The global max needs the whole tensor before
// any code can be written, so it takes two passes:
//   tensor_amax_kernel    per-block partial maxima (grid-stride over rows, 16-byte loads); block 0
//                         also saves the running amax as it was;
//   tensor_quant_kernel   each block reduces the partials to the scale (tensor_scale) and writes
//                         codes (any row count); or the TENSOR mode of the 128x128 dual kernel
//                         above when transposed codes are wanted as well.
// ---------------------------------------------------------------------------------------------
constexpr int kTensorRowsPerIter = 4;

// Visit (row, 8-column chunk) work items, rows strided by the grid and 4 rows per iteration so each
// thread keeps several 16-byte loads in flight.
template <typename TIn, typename F>
__device__ __forceinline__ void for_tensor_chunks(const TIn* x, int64_t R, int64_t C, int64_t ldx, F&& f) {
  const int64_t chunks = C / 8;
  for (int64_t r0 = (int64_t)blockIdx.x * kTensorRowsPerIter; r0 < R; r0 += (int64_t)gridDim.x * kTensorRowsPerIter) {
    for (int64_t c8 = threadIdx.x; c8 < chunks; c8 += blockDim.x) {
      float v[kTensorRowsPerIter][8];
#pragma unroll
      for (int i = 0; i < kTensorRowsPerIter; ++i)
        if (r0 + i < R) Load8<TIn>::run(x + (r0 + i) * ldx + 8 * c8, v[i]);
#pragma unroll
      for (int i = 0; i < kTensorRowsPerIter; ++i)
        if (r0 + i < R) f(r0 + i, 8 * c8, v[i]);
    }
  }
}

template <typename TIn>
__global__ __launch_bounds__(256) void tensor_amax_kernel(const TIn* __restrict__ x, int64_t R, int64_t C, int64_t ldx,
                                                          const float* __restrict__ amax, float* __restrict__ partial) {
  __shared__ float wmax[4];
  if (blockIdx.x == 0 && threadIdx.x == 0) partial[kTensorAmaxBlocks] = amax[0];
  float m = 0.0f;
  for_tensor_chunks(x, R, C, ldx, [&](int64_t, int64_t, const float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  });
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[blockIdx.x] = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

template <typename TIn, int FMT>
__global__ __launch_bounds__(256) void tensor_quant_kernel(const TIn* __restrict__ x, int64_t R, int64_t C,
                                                           int64_t ldx, TensorScaleArgs ta, uint8_t* __restrict__ q,
                                                           int64_t ldq) {
  const float sc = tensor_scale<TIn, FMT>(ta);
  const float rc = 1.0f / sc;
  for_tensor_chunks(x, R, C, ldx, [&](int64_t r, int64_t c, const float (&v)[8]) {
    float b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = sizeof(TIn) == 4 ? round_bf16(v[i]) : v[i];
    store_codes8(q + r * ldq + c, quant8<FMT, true>(b, sc, rc));
  });
}

// ---------------------------------------------------------------------------------------------
// Host launchers (arguments already validated; sizes non-empty).
// ---------------------------------------------------------------------------------------------
template <typename TIn, int FMT>
static hipError_t launch_1x128_t(const void* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                                 float* s, int64_t lds, hipStream_t st) {
  dim3 grid((unsigned)((R + kQ1Rows - 1) / kQ1Rows), (unsigned)(C / kGroup));
  hipLaunchKernelGGL((quant_1x128_kernel<TIn, FMT>), grid, dim3(256), 0, st, (const TIn*)x, R, ldx, q, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_quant_1x128(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, uint8_t* q,
                              int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  if (xt == 0)
    return fmt == kE4M3 ? launch_1x128_t<uint16_t, kE4M3>(x, R, C, ldx, q, ldq, s, lds, st)
                        : launch_1x128_t<uint16_t, kE5M2>(x, R, C, ldx, q, ldq, s, lds, st);
  return fmt == kE4M3 ? launch_1x128_t<float, kE4M3>(x, R, C, ldx, q, ldq, s, lds, st)
                      : launch_1x128_t<float, kE5M2>(x, R, C, ldx, q, ldq, s, lds, st);
}

template <typename TIn, int FMT>
static hipError_t launch_128x1_t(const void* x, int64_t R, int64_t C, int64_t ldx, uint8_t* qt, int64_t ldqt,
                                 float* st_, int64_t ldst, hipStream_t st) {
  const uint32_t ncg = (uint32_t)((C + kQtCols - 1) / kQtCols);
  hipLaunchKernelGGL((quant_128x1_kernel<TIn, FMT>), dim3((unsigned)(R / kGroup) * ncg), dim3(256), 0, st, (const TIn*)x,
                     C, ldx, qt, ldqt, st_, ldst, ncg);
  return hipGetLastError();
}

hipError_t launch_quant_128x1(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, uint8_t* qt,
                              int64_t ldqt, float* st_, int64_t ldst, hipStream_t st) {
  if (xt == 0)
    return fmt == kE4M3 ? launch_128x1_t<uint16_t, kE4M3>(x, R, C, ldx, qt, ldqt, st_, ldst, st)
                        : launch_128x1_t<uint16_t, kE5M2>(x, R, C, ldx, qt, ldqt, st_, ldst, st);
  return fmt == kE4M3 ? launch_128x1_t<float, kE4M3>(x, R, C, ldx, qt, ldqt, st_, ldst, st)
                      : launch_128x1_t<float, kE5M2>(x, R, C, ldx, qt, ldqt, st_, ldst, st);
}

template <typename TIn, int FR, int FC>
static hipError_t launch_dual_t(const void* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq, float* s,
                                int64_t lds, uint8_t* qt, int64_t ldqt, float* st_, int64_t ldst, hipStream_t st) {
  const uint32_t ncg = (uint32_t)(C / kQtCols);
  hipLaunchKernelGGL((quant_dual_kernel<TIn, FR, FC>), dim3((unsigned)(R / kGroup) * ncg), dim3(256), 0, st,
                     (const TIn*)x, ldx, q, ldq, s, lds, qt, ldqt, st_, ldst, ncg);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_dual_in(const void* x, int64_t R, int64_t C, int64_t ldx, int fr, uint8_t* q, int64_t ldq,
                                 float* s, int64_t lds, int fc, uint8_t* qt, int64_t ldqt, float* st_, int64_t ldst,
                                 hipStream_t st) {
  if (fr == kE4M3)
    return fc == kE4M3 ? launch_dual_t<TIn, kE4M3, kE4M3>(x, R, C, ldx, q, ldq, s, lds, qt, ldqt, st_, ldst, st)
                       : launch_dual_t<TIn, kE4M3, kE5M2>(x, R, C, ldx, q, ldq, s, lds, qt, ldqt, st_, ldst, st);
  return fc == kE4M3 ? launch_dual_t<TIn, kE5M2, kE4M3>(x, R, C, ldx, q, ldq, s, lds, qt, ldqt, st_, ldst, st)
                     : launch_dual_t<TIn, kE5M2, kE5M2>(x, R, C, ldx, q, ldq, s, lds, qt, ldqt, st_, ldst, st);
}

hipError_t launch_quant_dual(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fr, uint8_t* q,
                             int64_t ldq, float* s, int64_t lds, int fc, uint8_t* qt, int64_t ldqt, float* st_,
                             int64_t ldst, hipStream_t st) {
  if (xt == 0) return launch_dual_in<uint16_t>(x, R, C, ldx, fr, q, ldq, s, lds, fc, qt, ldqt, st_, ldst, st);
  return launch_dual_in<float>(x, R, C, ldx, fr, q, ldq, s, lds, fc, qt, ldqt, st_, ldst, st);
}

template <typename TIn, int FMT>
static hipError_t launch_128x128_t(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                                   float* s, int64_t lds, hipStream_t st) {
  const uint32_t nkb = (uint32_t)(K / kGroup);
  hipLaunchKernelGGL((quant_128x128_kernel<TIn, FMT>), dim3((unsigned)(N / kGroup) * nkb), dim3(256), 0, st,
                     (const TIn*)w, ldw, q, ldq, s, lds, nkb);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                                int64_t ldq, float* s, int64_t lds, hipStream_t st) {
  if (wt == 0)
    return fmt == kE4M3 ? launch_128x128_t<uint16_t, kE4M3>(w, N, K, ldw, q, ldq, s, lds, st)
                        : launch_128x128_t<uint16_t, kE5M2>(w, N, K, ldw, q, ldq, s, lds, st);
  return fmt == kE4M3 ? launch_128x128_t<float, kE4M3>(w, N, K, ldw, q, ldq, s, lds, st)
                      : launch_128x128_t<float, kE5M2>(w, N, K, ldw, q, ldq, s, lds, st);
}

template <typename TIn, int FMT>
static hipError_t launch_128x128_dual_t(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                                        float* s, int64_t lds, uint8_t* qt, int64_t ldqt, hipStream_t st) {
  const uint32_t nkb = (uint32_t)(K / kGroup);
  hipLaunchKernelGGL((quant_128x128_dual_kernel<TIn, FMT>), dim3((unsigned)(N / kGroup) * nkb), dim3(256), 0, st,
                     (const TIn*)w, ldw, q, ldq, s, lds, qt, ldqt, TensorScaleArgs{}, nkb);
  return hipGetLastError();
}

hipError_t launch_quant_128x128_dual(const void* w, int wt, int64_t N, int64_t K, int64_t ldw, int fmt, uint8_t* q,
                                     int64_t ldq, float* s, int64_t lds, uint8_t* qt, int64_t ldqt, hipStream_t st) {
  if (wt == 0)
    return fmt == kE4M3 ? launch_128x128_dual_t<uint16_t, kE4M3>(w, N, K, ldw, q, ldq, s, lds, qt, ldqt, st)
                        : launch_128x128_dual_t<uint16_t, kE5M2>(w, N, K, ldw, q, ldq, s, lds, qt, ldqt, st);
  return fmt == kE4M3 ? launch_128x128_dual_t<float, kE4M3>(w, N, K, ldw, q, ldq, s, lds, qt, ldqt, st)
                      : launch_128x128_dual_t<float, kE5M2>(w, N, K, ldw, q, ldq, s, lds, qt, ldqt, st);
}

template <typename TIn, int FMT>
static hipError_t launch_weights_dual_t(const WeightDualBatch& b, hipStream_t st) {
  hipLaunchKernelGGL((quant_weights_dual_kernel<TIn, FMT>), dim3(b.start[b.count]), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_quant_weights_dual(const WeightDualBatch& b, int wt, int fmt, hipStream_t st) {
  if (wt == 0)
    return fmt == kE4M3 ? launch_weights_dual_t<uint16_t, kE4M3>(b, st) : launch_weights_dual_t<uint16_t, kE5M2>(b, st);
  return fmt == kE4M3 ? launch_weights_dual_t<float, kE4M3>(b, st) : launch_weights_dual_t<float, kE5M2>(b, st);
}

// ---------------------------------------------------------------------------------------------
// Scratch for callers that cannot allocate (fp8bq_quantize_tensor_delayed_noalloc): the delayed
// quantizer's workspace (partial maxima and the saved running amax, kTensorWorkspace bytes) as a
// file-scope device array.  Each GPU holds its own copy for the life of the process, at its own
// address; host code uses that address, looked up once per device with the device current.  Nothing
// in it has to start at zero: every launch writes the parts it reads.  Calls that overlap on one GPU
// share it and race.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kTensorWorkspace / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
static std::atomic<float*> g_scratch[kMaxScratchDevices];

hipError_t tensor_scratch(int dev, float** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<float*>(a);
    g_scratch[dev].store(p, std::memory_order_release);  // (racing first calls store the same address)
  }
  *out = p;
  return hipSuccess;
}

int tensor_amax_blocks(int64_t R) {
  const int64_t want = (R + kTensorRowsPerIter - 1) / kTensorRowsPerIter;
  return (int)(want < kTensorAmaxBlocks ? (want > 0 ? want : 1) : kTensorAmaxBlocks);
}

template <typename TIn, int FMT>
static hipError_t launch_tensor_t(const void* x, int64_t R, int64_t C, int64_t ldx, float* amax, float b1, float b2,
                                  uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s, float* partial,
                                  hipStream_t st) {
  const int nb = tensor_amax_blocks(R);
  hipLaunchKernelGGL((tensor_amax_kernel<TIn>), dim3(nb), dim3(256), 0, st, (const TIn*)x, R, C, ldx,
                     (const float*)amax, partial);
  const hipError_t e = hipGetLastError();  // a failed launch stops the call before its second kernel
  if (e != hipSuccess) return e;
  const TensorScaleArgs ta{partial, nb, b1, b2, amax, s};
  if (qt) {
    const uint32_t ncg = (uint32_t)(C / kGroup);
    hipLaunchKernelGGL((quant_128x128_dual_kernel<TIn, FMT, true>), dim3((unsigned)(R / kGroup) * ncg), dim3(256), 0,
                       st, (const TIn*)x, ldx, q, ldq, s, (int64_t)0, qt, ldqt, ta, ncg);
  } else {
    hipLaunchKernelGGL((tensor_quant_kernel<TIn, FMT>), dim3(nb), dim3(256), 0, st, (const TIn*)x, R, C, ldx, ta, q,
                       ldq);
  }
  return hipGetLastError();
}

hipError_t launch_quant_tensor_delayed(const void* x, int xt, int64_t R, int64_t C, int64_t ldx, int fmt, float* amax,
                                       double beta, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s,
                                       void* ws, hipStream_t st) {
  const float b1 = (float)beta, b2 = (float)(1.0 - beta);
  float* partial = reinterpret_cast<float*>(ws);
  if (xt == 0)
    return fmt == kE4M3 ? launch_tensor_t<uint16_t, kE4M3>(x, R, C, ldx, amax, b1, b2, q, ldq, qt, ldqt, s, partial, st)
                        : launch_tensor_t<uint16_t, kE5M2>(x, R, C, ldx, amax, b1, b2, q, ldq, qt, ldqt, s, partial, st);
  return fmt == kE4M3 ? launch_tensor_t<float, kE4M3>(x, R, C, ldx, amax, b1, b2, q, ldq, qt, ldqt, s, partial, st)
                      : launch_tensor_t<float, kE5M2>(x, R, C, ldx, amax, b1, b2, q, ldq, qt, ldqt, s, partial, st);
}

}  // namespace fp8bq
