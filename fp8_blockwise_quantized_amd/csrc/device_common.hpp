// Device-side building blocks shared by the quantize and GEMM kernels (gfx950 / CDNA4).
//
// FP8 formats are the OCP ones the recipe names: E4M3 = float8_e4m3fn (max 448) and
// E5M2 = float8_e5m2 (max 57344) ("用 RTX 5090 花 $7000 训练 2B 大模型：Puro-2B 低成本预训练技术解析",
// section "Blackwell 的 FP8 Tensor Core").  gfx950's v_cvt_pk_{fp8,bf8}_f32 convert to exactly these
// formats with round-to-nearest-even.  A value above fmt_max but below the midpoint to the next
// binade step (464 for E4M3, 61440 for E5M2) rounds to the fmt_max code, as the quantize rule's
// clamp-then-convert gives; past that midpoint the converter gives NaN (E4M3) or Inf (E5M2), so a
// quotient that can get there is clamped first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

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

// Quotient x / s of a blockwise group, unclamped.  With |x| <= amax and s = RN(amax / fmt_max), the
// exact quotient is at most fmt_max / (1 - 2^-24) = fmt_max + 0.875 ulp(fmt_max) (fmt_max = 1.75 x a
// power of two), so its rounding is at most fmt_max + 1 ulp; with the floored scale it is below
// fmt_max.  The converter rounds fmt_max + 1 ulp (and its negative) to the fmt_max code, which is the
// clamped code, so the clamp changes no code and is left out (one VALU op per element and layout).
__device__ __forceinline__ float blockwise_quotient(float x, float s, float r) { return div_by_scale(x, s, r); }

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

// Four values -> one little-endian dword of codes (v0 in the lowest byte).  The first conversion
// writes the low half over v0's own bits (the high half is overwritten by the second), which spares
// a register clear per dword.
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float v0, float v1, float v2, float v3) {
  int w = cvt_pk<FMT, false>(v0, v1, __float_as_int(v0));
  w = cvt_pk<FMT, true>(v2, v3, w);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Lane exchanges within DPP rows (16 lanes).  Every pattern used here reads a valid lane for every
// lane, so bound_ctrl (zero for an invalid source) never applies; with old = 0 it lets the compiler
// fold the move into the consuming max as one v_max_u32_dpp.
constexpr int kDppXor8 = 0x128;    // row_ror:8: partner lane ^ 8
constexpr int kDppMirror8 = 0x141; // row_half_mirror: partner 7 - lane within each half row
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]: partner lane ^ 2
constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]: partner lane ^ 1
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_read(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// Max of non-negative finite floats (or +0) held as bits: their order is the unsigned integer order.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint32_t umax_partner(uint32_t mine, uint32_t sent) {
  return umax(mine, dpp_read<CTRL>(sent));
}

// Max over the 16 lanes of each DPP row (all 16 lanes receive it).  Values are >= 0.
__device__ __forceinline__ float row16_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax_partner<kDppXor8>(u, u);
  u = umax_partner<kDppMirror8>(u, u);
  u = umax_partner<kDppXor2>(u, u);
  u = umax_partner<kDppXor1>(u, u);
  return __uint_as_float(u);
}

// Reduce-scatter over a DPP row: each of the 16 lanes holds partial maxima m[0..NR) of the same NR
// rows (NR = 1, 2, 4 or 8; values >= 0 as bits).  Stage S exchanges with the partner that differs
// in lane bit 3 - S; while more than one row is left, a lane keeps the half of its rows picked by
// that bit and sends the other half, so the rows halve at each stage; the remaining stages take the
// plain max.  On return lane l holds the 16-lane max of row (l >> (4 - log2 NR)) & (NR - 1), and
// row r sits in lane r << (4 - log2 NR) (and the lanes up to the next such lane).
template <int S>
constexpr int scatter_ctrl() {
  return S == 0 ? kDppXor8 : S == 1 ? kDppMirror8 : S == 2 ? kDppXor2 : kDppXor1;
}
template <int S, int N, int NR>
__device__ __forceinline__ void scatter_stage(uint32_t (&a)[NR], int lane16) {
  if constexpr (S < 4) {
    if constexpr (N > 1) {
      const bool hi = (lane16 >> (3 - S)) & 1;
#pragma unroll
      for (int k = 0; k < N / 2; ++k) {
        const uint32_t keep = hi ? a[k + N / 2] : a[k];
        const uint32_t send = hi ? a[k] : a[k + N / 2];
        a[k] = umax_partner<scatter_ctrl<S>()>(keep, send);
      }
      scatter_stage<S + 1, N / 2>(a, lane16);
    } else {
      a[0] = umax_partner<scatter_ctrl<S>()>(a[0], a[0]);
      scatter_stage<S + 1, 1>(a, lane16);
    }
  }
}
template <int NR>
__device__ __forceinline__ float row16_max_scatter(const float (&m)[NR], int lane16) {
  static_assert(NR == 1 || NR == 2 || NR == 4 || NR == 8, "rows per lane");
  uint32_t a[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) a[k] = __float_as_uint(m[k]);
  scatter_stage<0, NR>(a, lane16);
  return __uint_as_float(a[0]);
}
// log2 of the lanes that share one row after row16_max_scatter<NR>.
template <int NR>
constexpr int scatter_shift() {
  return NR == 8 ? 1 : NR == 4 ? 2 : NR == 2 ? 3 : 4;
}
// Value of lane LANE of this lane's DPP row (row_newbcast).
template <int LANE>
__device__ __forceinline__ float row16_bcast(float v) {
  static_assert(LANE >= 0 && LANE < 16, "lane");
  return __uint_as_float(dpp_read<0x150 + LANE>(__float_as_uint(v)));
}

// Max over the whole 64-lane wavefront (uniform result).  Values are >= 0.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order (a compile-time index, for
// operands that must be constants such as DPP controls).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
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
