// Device-side building blocks shared by the quantize and GEMM kernels (gfx950 / CDNA4).
//
// FP8 formats are the OCP ones the recipe names: E4M3 = float8_e4m3fn (max 448) and
// E5M2 = float8_e5m2 (max 57344) ("用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析",
// section "Blackwell 的 FP8 Tensor Core").  gfx950's v_cvt_pk_{fp8,bf8}_f32 convert to exactly these
// formats with round-to-nearest-even; the quantizer clamps to +-fmt_max first, so the converter never
// sees an out-of-range value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bq {

constexpr int kGroup = 128;  // every scale block is 128 wide along its grouped axis

enum Fmt : int { kE4M3 = 0, kE5M2 = 1 };

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<kE4M3> {
  static constexpr float kMax = 448.0f;
};
template <>
struct FmtTraits<kE5M2> {
  static constexpr float kMax = 57344.0f;
};

// fp32(1e-12): the scale floor of the quantize rule.
__device__ __forceinline__ float scale_floor() { return __uint_as_float(0x2B8CBCCCu); }

// Scale of one group: IEEE fp32 amax / fmt_max (hipcc's default '/' is correctly rounded),
// floored at fp32(1e-12).
template <int FMT>
__device__ __forceinline__ float group_scale(float amax) {
  float s = amax / FmtTraits<FMT>::kMax;
  return s < scale_floor() ? scale_floor() : s;
}

// Correctly rounded fp32 quotient x / s given r = RN(1/s).
// Markstein's division theorem: if r is within half an ulp of 1/s and q0 = RN(x*r) is within one ulp
// of x/s, the residual e = q0*s - x is exact (one fused multiply-add) and RN(q0 - e*r) is the
// correctly rounded quotient.  The residual is taken with this sign so that x = -0 gives -0.
// Exactness of e fails only for |x| below about 2^-100; since s >= 1e-12 such quotients are below
// 2^-60, far under the smallest FP8 rounding boundary (2^-17), so they encode to the same signed zero
// as the IEEE quotient and the codes still match an IEEE division bit for bit.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}

template <int FMT>
__device__ __forceinline__ float clamp_fmt(float y) {
  return __builtin_fminf(__builtin_fmaxf(y, -FmtTraits<FMT>::kMax), FmtTraits<FMT>::kMax);
}

// Two clamped fp32 values -> two FP8 codes in the low (hi=false) or high (hi=true) 16 bits of `old`.
template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pk(float a, float b, int old) {
  if constexpr (FMT == kE4M3)
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else
    return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// Four values -> one little-endian dword of codes (v0 in the lowest byte).
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float v0, float v1, float v2, float v3) {
  int w = cvt_pk<FMT, false>(v0, v1, 0);
  w = cvt_pk<FMT, true>(v2, v3, w);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Max over the 16 lanes of each DPP row (all 16 lanes receive it).  Values are >= 0.
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
  return v;
}

// Max over the whole 64-lane wavefront (uniform result).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

// Round-to-nearest-even fp32 -> bf16 pair, lo in the low half: one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Tile (row, column) of a block of a 2-D tile grid launched in one dimension (up to 2^31 blocks; a
// grid's second dimension is much shorter), column tiles fastest as a 2-D grid would dispatch them.
struct TileRC {
  int64_t row, col;
};
__device__ __forceinline__ TileRC tile_of_block(uint32_t ncols) {
  const uint32_t b = blockIdx.x;
  const uint32_t r = b / ncols;
  return TileRC{(int64_t)r, (int64_t)(b - r * ncols)};
}

// fp32 value of the nearest BF16 number (ties to even).
__device__ __forceinline__ float round_bf16(float v) { return bf16lo(pack_bf16x2(v, 0.0f)); }

}  // namespace fp8bq
