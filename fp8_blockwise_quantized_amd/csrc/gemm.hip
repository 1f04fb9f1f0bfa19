// Scaled FP8 GEMM for gfx950 (CDNA4): fprop, dgrad and wgrad of the blockwise-quantized linear layer.
//
// The product ("小团队也能预训练！普罗2B：RTX5090训练成本不到5090美元", paragraph
// "FP8发挥RTX 5090的低精度效率优势"; "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090",
// "方法关键点", bullet "FP8 blockwise 混合精度") is, in the kernel's TN frame,
//     C[m, n] = sum_kb sa(kb, m) * sb(kb, n) * sum_{k in kb} dec(A[m, k]) * dec(B[n, k])
// with FP32 accumulation and BF16 (or FP32) output.  One v_mfma_f32_16x16x128_f8f6f4 covers exactly
// one 128-long scale block of the contraction for a 16x16 output patch, so the kernel issues each
// MFMA with a zero accumulator and folds its result into the running FP32 sum with one FMA per
// output element: acc += mfma * (sa * sb).  Mixed formats (E5M2 gradients x E4M3 weights) are the
// instruction's per-operand format fields.
//
// Operand roles: the MFMA's first operand is the B patch (16 output columns) and its second the A
// patch (16 output rows).  A lane then holds output row (lane % 16) and four output columns of the B
// patch, so the A-side scale is one value per lane and patch.  For fprop and dgrad the B patches'
// rows are permuted so that a lane holds runs of 8 consecutive columns and the 4 lanes of an output
// row hold 32 consecutive columns: the epilogue writes 64 contiguous bytes of BF16 per row and store.
//
// Data movement: per 128-long contraction block the workgroup stages a BM x 128 A tile and a
// BN x 128 B tile in LDS (double-buffered, one barrier per block), with 16-byte chunks XOR-swizzled
// by row so the 16-byte fragment reads of 64 lanes spread over all banks.  Global loads for block
// kb+1 (and its scales) are issued before the MFMAs of block kb.  Workgroup ids are remapped so that
// each XCD (its own L2) works on a contiguous, row-grouped region of output tiles.

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8bq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzle inside a 128-byte LDS row.  It depends on row % 16 only, so every 16-row
// patch has the same per-lane read pattern (one pair of lane offsets serves all patches; the patch
// position goes into the instruction's immediate offset).  Conflict-free for 8-lane phases (rows
// 0-7 and 8-15 each get 8 distinct chunks) and for 16-lane phases over 64 banks (rows of equal
// parity get distinct chunks).
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

constexpr int kGroupRows = 8;  // output tile rows per L2 group
constexpr int kXcds = 8;

// Bijective remap of the hardware workgroup id (dispatched round-robin over the XCDs) to a logical
// tile id so each XCD processes a contiguous range of logical ids, then row-grouped tile ordering.
// 32-bit arithmetic (the planner keeps tile and unit counts below 2^31); the results are wave-uniform
// and kept in scalar registers.
__device__ __forceinline__ void tile_of(uint32_t w, uint32_t tiles_m, uint32_t tiles_n, uint32_t& tm, uint32_t& tn) {
  const uint32_t nblk = tiles_m * tiles_n;
  const uint32_t q8 = nblk / kXcds, r8 = nblk % kXcds;
  const uint32_t x = w % kXcds;
  const uint32_t L = x * q8 + (x < r8 ? x : r8) + w / kXcds;
  const uint32_t group = (uint32_t)kGroupRows * tiles_n;
  const uint32_t gid = L / group;
  const uint32_t first = gid * kGroupRows;
  const uint32_t gsz = (tiles_m - first) < (uint32_t)kGroupRows ? (tiles_m - first) : (uint32_t)kGroupRows;
  const uint32_t rem = L - gid * group;
  tm = __builtin_amdgcn_readfirstlane(first + rem % gsz);
  tn = __builtin_amdgcn_readfirstlane(rem / gsz);
}

template <int FA, int FB>
__device__ __forceinline__ v4f mfma_block(const v8i& bpatch, const v8i& apatch) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = format of the first operand (B patch), blgp = format of the second (A patch);
  // zero E8M0 scale operands select the unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bpatch, apatch, zero, FB, FA, 0, 0, 0, 0);
}

// Byte offsets, within a 16-row patch, of the two 16-byte chunks lane reads: row lane % 16, logical
// chunks 2*(lane/16) and 2*(lane/16)+1 (32 consecutive contraction bytes).
struct PatchLane {
  int lo, hi;
};
__device__ __forceinline__ PatchLane patch_lane(int lane) {
  const int r = lane & 15, s = swz(r), c0 = 2 * (lane >> 4);
  return PatchLane{r * 128 + ((c0 ^ s) << 4), r * 128 + (((c0 + 1) ^ s) << 4)};
}
// B-side patches are permuted: row rho of B patch j (a wave's four patches of 16 output columns)
// is output column 8*(rho/4) + 32*(j/2) + 4*(j%2) + rho%4 of the wave's 64 columns.  Lane l then
// holds, for patches 2t and 2t+1, the 8 consecutive columns 32*t + 8*(l/16) .. +7 of its output row,
// so the four lanes of a row write 64 contiguous bytes per store.  B tile rows get their own chunk
// swizzle: lane l's row 8*(rho/4) + rho%4 (rho = l % 16) takes the swizzle A-side row rho has, so
// every lane of a B-patch read hits exactly the bank of the same lane's A-patch read, and the two
// reads conflict alike on any grouping of lanes into LDS phases (A's pattern is conflict-free).  It
// ignores row bit 2 and bits 5 and up, so it is the same for all four patches (their rows differ by
// 32*(j/2) + 4*(j%2)) and for every wave column.
__device__ __forceinline__ int swzb(int row) { return swz(4 * ((row >> 3) & 3) + (row & 3)); }
__device__ __forceinline__ PatchLane b_patch_lane(int lane) {
  const int rho = lane & 15, r = 8 * (rho >> 2) + (rho & 3), s = swzb(r), c0 = 2 * (lane >> 4);
  return PatchLane{r * 128 + ((c0 ^ s) << 4), r * 128 + (((c0 + 1) ^ s) << 4)};
}
// The MFMA operand of the 16-row patch starting at patch_base (a multiple of 16 rows into a tile).
__device__ __forceinline__ v8i lds_patch(const uint8_t* patch_base, PatchLane pl) {
  const v4i lo = *reinterpret_cast<const v4i*>(patch_base + pl.lo);
  const v4i hi = *reinterpret_cast<const v4i*>(patch_base + pl.hi);
  v8i r = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor over [base, base + bytes): loads past the end read zeros instead of
// faulting.  Word 3 is the gfx9 raw-buffer format word.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ uint32_t sat32(int64_t bytes) {
  return bytes < 0 ? 0u : (bytes < (int64_t)0xFFFFFFFF ? (uint32_t)bytes : 0xFFFFFFFFu);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// One 16-byte (or 4-byte) load per lane from byte offset voff of the buffer, written straight into
// LDS at lds_base + 16 * lane (or 4 * lane): buffer_load_dwordx4 / _dword with the lds flag.
// lds_base must be the same for the whole wave.  (Buffer loads rather than global_load_lds: the
// compiler then keeps exact counts for the waits on LDS reads.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, 0, 0, 0);
}

// One work unit: an output tile and the range of 128-long contraction blocks it sums.
struct Unit {
  int m0, n0;
  int kb0, kb1, split;
};

template <int BM, int BN>
__device__ __forceinline__ Unit unit_of(uint32_t u, uint32_t tiles_m, uint32_t tiles_n, int nsplit, int nkb) {
  const uint32_t T = tiles_m * tiles_n;
  const uint32_t w = u % T;
  const int s = (int)(u / T);
  uint32_t tm, tn;
  tile_of(w, tiles_m, tiles_n, tm, tn);
  Unit r;
  r.m0 = (int)tm * BM;
  r.n0 = (int)tn * BN;
  r.kb0 = __builtin_amdgcn_readfirstlane(s * nkb / nsplit);
  r.kb1 = __builtin_amdgcn_readfirstlane((s + 1) * nkb / nsplit);
  r.split = __builtin_amdgcn_readfirstlane(s);
  return r;
}

// OP (fprop / dgrad / wgrad) only names the instance, so profiles attribute time per product.
//
// Persistent workgroups: workgroup b processes work units b, b + G, b + 2G, ... (G = grid size, a
// multiple of 8 when there is more than one round, so every unit of a workgroup maps to its XCD's
// contiguous range in tile_of).  A unit is one BM x BN output tile and a range of contraction blocks
// (all of them, or 1/nsplit when the contraction is split; split units write FP32 partial sums that
// a separate pass adds in a fixed order).  The LDS ring runs continuously across units: the loads
// for a unit's first block are issued while the previous unit's last block is multiplied and its
// tile is written out.
//
// LDS stage layout (NSTAGE stages, a ring): [A tile BM x 128 B][B tile BN x 128 B][A scales BM x f32]
// [B scales: BN x f32 (per-column mode) or one f32 per 128 columns (per-block mode), 64 slots min]
// [256 B sink for padding loads].  Tiles and scales arrive by direct global->LDS loads: wave w fills
// 1 KB chunks w, w+NW, ... (8 rows each); lane l of a chunk fetches the 16 bytes that belong at LDS
// offset 16*l, i.e. row l/8 and physical chunk l%8, whose logical chunk is (l%8) ^ swz(row).  Every
// wave issues the same number of loads per stage (scale jobs are padded with loads into the sink), so
// one s_waitcnt vmcnt(loads per stage) leaves exactly the newest stage in flight.
// Workgroups per CU that the LDS ring allows for a 4-wave tile (the planner's slots per CU: four for
// 64x64, two for 128x128); the launch bound then keeps the registers low enough for that residency.
template <int BM, int BN, int NW, int NSTAGE>
struct StageMinBlocks {
  static constexpr int kStage = (BM + BN) * 128 + BM * 4 + 64 * 4 + 256;  // lower bound of STAGE
  static constexpr int value = NW != 4 ? 1 : 4 * NSTAGE * kStage <= 160 * 1024 ? 4 : 2 * NSTAGE * kStage <= 160 * 1024 ? 2 : 1;
};

template <int OP, int BM, int BN, int WGM, int WGN, int NSTAGE, int SBM, int FA, int FB, int OUTF32>
__global__ __launch_bounds__(WGM* WGN * 64, (StageMinBlocks<BM, BN, WGM * WGN, NSTAGE>::value)) void gemm_tn_kernel(
    GemmDesc d, uint32_t tiles_m, uint32_t tiles_n, int nsplit, float* __restrict__ partial) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM;
  constexpr int WTN = BN / WGN;
  constexpr int MI = WTM / 16;
  constexpr int NI = WTN / 16;
  constexpr int SA_OFF = (BM + BN) * 128;
  constexpr int NSB = SBM == kSbColumn ? BN : ((BN + kGroup - 1) / kGroup);  // (a 64-wide tile: one block)
  constexpr int SB_OFF = SA_OFF + BM * 4;
  constexpr int SINK_OFF = SB_OFF + (NSB > 64 ? NSB : 64) * 4;
  constexpr int STAGE = SINK_OFF + 256;
  constexpr int ACHUNKS = BM / 8, BCHUNKS = BN / 8;  // 1 KB chunks per stage
  constexpr int SAJOBS = BM / 64;                     // 64 scales per wave job
  constexpr int SBJOBS = NSB > 64 ? NSB / 64 : 1;
  constexpr int SJOBS = SAJOBS + SBJOBS;
  constexpr int JPW = (SJOBS + NW - 1) / NW;          // scale jobs per wave (padded)
  // B patch rows permuted for 16-byte BF16 stores (fprop / dgrad); the per-column-scale product
  // (wgrad), mostly written as FP32 partial sums, keeps natural order (64-byte FP32 runs per row)
  constexpr bool PERM = SBM == kSbBlock128;
  static_assert(!PERM || NI == 4, "the B-side permutation is laid out for 64-column wave tiles");
  constexpr int LOADS = ACHUNKS / NW + BCHUNKS / NW + JPW;  // loads per wave per stage
  static_assert(ACHUNKS % NW == 0 && BCHUNKS % NW == 0, "tile chunks must split evenly over waves");
  static_assert(BM % 64 == 0 && (NSB <= 64 || NSB % 64 == 0), "scale jobs are 64 lanes wide");
  static_assert(SBM != kSbBlock128 || WTN <= 128, "a wave's columns must share one weight block");
  static_assert(SBM != kSbBlock128 || BN % kGroup == 0 || kGroup % BN == 0, "a narrow tile lies in one weight block");
  static_assert(NSTAGE >= 2 && NSTAGE * STAGE <= 160 * 1024, "LDS ring does not fit");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wid / WGN, wn = wid % WGN;
  const int64_t M = d.M, N = d.N;
  const int nkb = (int)(d.K / kGroup);
  const uint32_t U = tiles_m * tiles_n * (uint32_t)nsplit;
  const uint32_t G = gridDim.x;

  // load-side cursor: unit lu, block lkb, and this lane's sources for that unit as 32-bit offsets
  // from workgroup-uniform bases (rows past the end are clamped; their results are never stored)
  uint32_t lu = blockIdx.x;
  Unit L = unit_of<BM, BN>(lu, tiles_m, tiles_n, nsplit, nkb);
  int lkb = L.kb0;
  bool lmore = true;
  const uint8_t* abase = d.a;
  const uint8_t* bbase = d.b;
  uint32_t abytes = 0, bbytes = 0;  // from abase / bbase to the end of the tile's last valid row
  uint32_t aoff[ACHUNKS / NW], boff[BCHUNKS / NW];
  const float* gs[JPW];  // scale job q: array base (wave-uniform), per-lane byte offset, kb stride
  int64_t gsk[JPW];
  uint32_t gsbytes[JPW];
  uint32_t gvo[JPW];
  int lso[JPW];
  auto set_sources = [&](const Unit& u) {
    abase = d.a + (int64_t)u.m0 * d.lda;
    bbase = d.b + (int64_t)u.n0 * d.ldb;
    const int64_t mleft = M - 1 - u.m0, nleft = N - 1 - u.n0;
    abytes = sat32((mleft < BM - 1 ? mleft : BM - 1) * d.lda + d.K);
    bbytes = sat32((nleft < BN - 1 ? nleft : BN - 1) * d.ldb + d.K);
#pragma unroll
    for (int i = 0; i < ACHUNKS / NW; ++i) {
      const int row = 8 * (wid + NW * i) + (lane >> 3);
      const int64_t r = row < mleft ? row : mleft;
      aoff[i] = (uint32_t)(r * d.lda) + (uint32_t)(((lane & 7) ^ swz(row)) * 16);
    }
#pragma unroll
    for (int i = 0; i < BCHUNKS / NW; ++i) {
      const int row = 8 * (wid + NW * i) + (lane >> 3);
      const int64_t r = row < nleft ? row : nleft;
      boff[i] = (uint32_t)(r * d.ldb) + (uint32_t)(((lane & 7) ^ (PERM ? swzb(row) : swz(row))) * 16);
    }
    // scale jobs: job j < SAJOBS loads A scales of rows 64j..64j+63, the next SBJOBS the B scales;
    // wave w runs jobs w, w+NW, ...; missing jobs load a valid scale into the sink
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
      const int j = wid + NW * q;
      if (j < SAJOBS) {
        int64_t m = u.m0 + 64 * j + lane;
        m = m < M ? m : M - 1;
        gs[q] = d.sa;
        gvo[q] = (uint32_t)(m * 4 * d.sa_mstride);
        gsk[q] = d.ldsa;
        gsbytes[q] = d.sa_mstride ? sat32(M * 4) : 4;
        lso[q] = SA_OFF + 256 * j;
      } else if (j < SJOBS) {
        const int v = j - SAJOBS;
        gs[q] = d.sb;
        if constexpr (SBM == kSbColumn) {
          int64_t n = u.n0 + 64 * v + lane;
          n = n < N ? n : N - 1;
          gvo[q] = (uint32_t)(n * 4);
          gsbytes[q] = sat32(N * 4);
        } else {
          const int64_t nbl = N / kGroup;
          int64_t nb = u.n0 / kGroup + (lane < NSB ? lane : NSB - 1);
          nb = nb < nbl ? nb : nbl - 1;
          gvo[q] = (uint32_t)(nb * d.sb_nstride * 4);
          gsbytes[q] = sat32(((nbl - 1) * d.sb_nstride + 1) * 4);
        }
        gsk[q] = d.sb_kstride;
        lso[q] = SB_OFF + 256 * v;
      } else {
        gs[q] = d.sa;
        gvo[q] = 0;
        gsk[q] = 0;
        gsbytes[q] = 4;
        lso[q] = SINK_OFF;
      }
    }
  };
  // Issue the loads of (lu, lkb) into stg, then advance the cursor.  Once every block has been
  // issued the cursor stays on the last one and further calls load it again into the free slot:
  // every call issues exactly LOADS loads, so one constant s_waitcnt serves every iteration and no
  // branch separates the MFMAs from their folds.  (A slot refilled that way is never read: it would
  // hold a block past the end.)
  // load number i (0 <= i < LOADS) of this wave for the current cursor position
  auto issue_load = [&](int i, uint8_t* stg) {
    if (i < ACHUNKS / NW) {
      dma16(rsrc_of(abase + lkb * kGroup, abytes - (uint32_t)(lkb * kGroup)), aoff[i], stg + (wid + NW * i) * 1024);
    } else if (i < ACHUNKS / NW + BCHUNKS / NW) {
      const int b = i - ACHUNKS / NW;
      dma16(rsrc_of(bbase + lkb * kGroup, bbytes - (uint32_t)(lkb * kGroup)), boff[b],
            stg + BM * 128 + (wid + NW * b) * 1024);
    } else {
      const int q = i - ACHUNKS / NW - BCHUNKS / NW;
      dma4(rsrc_of(gs[q] + (int64_t)lkb * gsk[q], gsbytes[q]), gvo[q], stg + lso[q]);
    }
  };
  auto advance = [&]() {
    if (lmore && ++lkb == L.kb1) {
      if (lu + G < U) {
        lu += G;
        L = unit_of<BM, BN>(lu, tiles_m, tiles_n, nsplit, nkb);
        lkb = L.kb0;
        set_sources(L);
      } else {
        lkb = L.kb1 - 1;
        lmore = false;
      }
    }
  };
  auto load_next = [&](uint8_t* stg) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) issue_load(i, stg);
    advance();
  };
  // Every wave waits for its own loads of the next block, then the barrier makes them (and the end
  // of all reads of the current block's slot) visible workgroup-wide.  No memory fence: loads of
  // the blocks after the next stay in flight across the barrier.
  auto stage_barrier = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((NSTAGE - 2) * LOADS) : "memory");
  };

  v4f acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  if (lu >= U) return;  // (the grid never exceeds the unit count)
  set_sources(L);
  // compute-side cursor
  uint32_t cu = lu;
  Unit C = L;
  int ckb = C.kb0;

  // The side with fewer 16-row patches stays in registers for the whole block ("resident"); the
  // other side is streamed one patch at a time.  MFMA order: streamed patch outer, except for the
  // last TAILN streamed patches (the tail), which alternate (resident patch outer) so that resident
  // patch k is free after MFMA TAILN*k + TAILN-1 of the tail.
  constexpr bool STREAM_B = NI > MI;
  constexpr int NOUT = STREAM_B ? NI : MI;  // streamed patches
  constexpr int NIN = STREAM_B ? MI : NI;   // resident patches
  constexpr int NTILE = MI * NI;
  // MFMA u is folded LAG steps after its issue.  Three steps leave the result complete before the
  // fold reads it (the compiler's VALU-after-MFMA wait states drop from 13 to 3 per block, +2-4% on
  // fprop/dgrad); wgrad, whose fold is twice as long and whose registers are fuller, keeps two.
  constexpr int LAG = SBM == kSbBlock128 ? 3 : 2;
#ifndef FP8BQ_TAILN
#define FP8BQ_TAILN 3
#endif
  constexpr int TAILN = (PERM && NOUT >= 6) ? FP8BQ_TAILN : 2;  // streamed patches in the tail
  constexpr int TAIL0 = (NOUT - TAILN) * NIN;  // first MFMA of the tail
  constexpr int UB = TAIL0 + TAILN - 1;        // step that ends with the stage barrier
  constexpr int NPOST = NTILE + LAG - UB - 1;  // steps after it
  static_assert(NOUT >= TAILN && NPOST >= 1, "tile too small for the pipelined order");
  auto order = [&](int u, int& o, int& k) {
    if (u < TAIL0) {
      o = u / NIN;
      k = u % NIN;
    } else {
      o = NOUT - TAILN + (u - TAIL0) % TAILN;
      k = (u - TAIL0) / TAILN;
    }
  };
  const PatchLane pl = patch_lane(lane);
  const PatchLane plb = PERM ? b_patch_lane(lane) : pl;
  auto apatch = [&](const uint8_t* stg, int i) { return lds_patch(stg + wm * WTM * 128 + 16 * i * 128, pl); };
  auto bpatch = [&](const uint8_t* stg, int j) {
    return lds_patch(stg + BM * 128 + wn * WTN * 128 + (PERM ? (4096 * (j >> 1) + 512 * (j & 1)) : 2048 * j), plb);
  };
  auto streamed = [&](const uint8_t* stg, int o) { return STREAM_B ? bpatch(stg, o) : apatch(stg, o); };
  auto resident = [&](const uint8_t* stg, int k) { return STREAM_B ? apatch(stg, k) : bpatch(stg, k); };
  // Streamed patches are read RA patches ahead of their first MFMA (two where the registers allow).
  constexpr int RA = (PERM && NOUT >= 3) ? 2 : 1;
  // The next block's first reads (its resident patches and first RA streamed patches), in the order
  // the current block's tail frees their registers: read h goes out at tail step 2 + 2h.
  constexpr int NHEAD = NIN + RA;
  auto head_read = [&](const uint8_t* stg, int h, v8i* res, v8i* str) {
    if (h == 0) res[0] = resident(stg, 0);
    else if (h <= RA) str[h - 1] = streamed(stg, h - 1);
    else res[h - RA] = resident(stg, h - RA);
  };

  // prologue: every ring slot's block in flight, the first landed, its first reads issued
  v8i res[NIN], str[NOUT];
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) load_next(smem + s * STAGE);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((NSTAGE - 1) * LOADS) : "memory");
#pragma unroll
  for (int h = 0; h < NHEAD; ++h) head_read(smem, h, res, str);

  int rd = 0;  // ring slot of the block multiplied this iteration
  while (true) {
    const int nx = rd + 1 == NSTAGE ? 0 : rd + 1;
    const uint8_t* stage = smem + rd * STAGE;
    const uint8_t* nstage = smem + nx * STAGE;

    // Step u issues MFMA u (and the read-ahead of the next streamed patch) and the fold of MFMA
    // u-LAG, whose result is then complete; a scheduling fence closes every step, so the matrix pipe
    // never waits on a fold and at most LAG+1 MFMA results are live.  Step UB ends with the stage
    // barrier: every wave has read all it needs of this block (the tail's operands are in registers)
    // and the next block has landed.  The steps after it refill this block's slot with the block
    // NSTAGE ahead and read the next block's first patches while the tail's MFMAs run.
    const float* ssa = reinterpret_cast<const float*>(stage + SA_OFF);
    const float* ssb = reinterpret_cast<const float*>(stage + SB_OFF);
    float sa_[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) sa_[i] = ssa[wm * WTM + 16 * i + (lane & 15)];
    float sbv = 0.0f;
    v4f sbc[NI];
    if constexpr (SBM == kSbBlock128) {
      sbv = ssb[(wn * WTN) / kGroup];
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j)
        sbc[j] = *reinterpret_cast<const v4f*>(ssb + wn * WTN + 16 * j + 4 * (lane >> 4));
    }
    v4f p[NTILE];
    // Several workgroups per CU (one wave of each per SIMD): a wave runs its MFMA steps at raised
    // priority and drops back at the stage barrier, so the workgroups drift out of phase instead of
    // contending for the matrix pipe and the refill at the same time (+6% on a 128x128-tile wgrad;
    // neutral with one workgroup per CU, where it is not used).
    constexpr bool PRIO = StageMinBlocks<BM, BN, NW, NSTAGE>::value >= 2;
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NTILE + LAG; ++u) {
      if (u < NTILE) {
        int o, k;
        order(u, o, k);
        if (k == 0 && o + RA < NOUT) str[o + RA] = streamed(stage, o + RA);
        p[u] = STREAM_B ? mfma_block<FA, FB>(str[o], res[k]) : mfma_block<FA, FB>(res[k], str[o]);
      }
      if (u == UB) {
        stage_barrier();
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      }
      if (u > UB) {
        const int t = u - UB - 1;  // post-barrier step 0 .. NPOST-1
#pragma unroll
        for (int i = t * LOADS / NPOST; i < (t + 1) * LOADS / NPOST; ++i) issue_load(i, smem + rd * STAGE);
      }
      if (u >= UB && (u - UB) % 2 == 1 && (u - UB) / 2 < NHEAD) head_read(nstage, (u - UB) / 2, res, str);
      if (u >= LAG) {
        int o, k;
        order(u - LAG, o, k);
        const int v = u - LAG;
        const int i = STREAM_B ? k : o, j = STREAM_B ? o : k;
        if constexpr (SBM == kSbBlock128) {
          const float sc = sa_[i] * sbv;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[v][r], sc, acc[i][j][r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[v][r], sa_[i] * sbc[j][r], acc[i][j][r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // head reads that did not fit into the steps
#pragma unroll
    for (int h = 0; h < NHEAD; ++h)
      if (UB + 1 + 2 * h >= NTILE + LAG) head_read(nstage, h, res, str);
    // keep the folds in the step sequence (not sunk past the cursor update's branches)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) asm volatile("" : "+v"(acc[i][j]));
    advance();
    rd = nx;

    if (++ckb < C.kb1) continue;

    // unit finished: write the tile (or its partial sum) and move on.  Lane l holds row l % 16 of
    // each 16-row A patch and, of the wave's 64 columns, 8*(l/16) + 32*(j/2) + 4*(j%2) .. +3 for
    // patch j (permuted B rows) or 16*j + 4*(l/16) .. +3 (natural order); only tiles that reach past
    // M or N check bounds.
    {
      const int64_t mrow = (int64_t)C.m0 + wm * WTM + (lane & 15);
      const int64_t ncol = (int64_t)C.n0 + wn * WTN + (PERM ? 8 : 4) * (lane >> 4);
      auto jcol = [](int j) { return PERM ? 32 * (j >> 1) + 4 * (j & 1) : 16 * j; };  // patch j's offset from ncol
      const bool full = (int64_t)C.m0 + BM <= M && (int64_t)C.n0 + BN <= N;
      auto write = [&](auto checked) {
        constexpr bool CHK = decltype(checked)::value;
        if (nsplit > 1 || OUTF32) {
          const int64_t ldc = nsplit > 1 ? N : d.ldc;
          float* c0 = (nsplit > 1 ? partial + (int64_t)C.split * M * N : reinterpret_cast<float*>(d.c)) + mrow * ldc + ncol;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            float* ci = c0 + 16 * i * ldc;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
              if (CHK && !(mrow + 16 * i < M && ncol + jcol(j) < N)) continue;
              v4f* cij = reinterpret_cast<v4f*>(ci + jcol(j));
              if (OUTF32 == 2 && nsplit == 1)
                *cij = *cij + acc[i][j];
              else
                *cij = acc[i][j];
            }
          }
        } else if constexpr (PERM) {
          uint16_t* c0 = reinterpret_cast<uint16_t*>(d.c) + mrow * d.ldc + ncol;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            uint16_t* ci = c0 + 16 * i * d.ldc;
#pragma unroll
            for (int t = 0; t < NI / 2; ++t) {
              if (CHK && !(mrow + 16 * i < M && ncol + 32 * t < N)) continue;
              const v4f& a = acc[i][2 * t];
              const v4f& b = acc[i][2 * t + 1];
              *reinterpret_cast<uint4*>(ci + 32 * t) = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                                   pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
            }
          }
        } else {
          uint16_t* c0 = reinterpret_cast<uint16_t*>(d.c) + mrow * d.ldc + ncol;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            uint16_t* ci = c0 + 16 * i * d.ldc;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
              if (CHK && !(mrow + 16 * i < M && ncol + 16 * j < N)) continue;
              *reinterpret_cast<uint2*>(ci + 16 * j) =
                  make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
            }
          }
        }
      };
      if (full) {
        write(std::false_type{});
      } else {
        write(std::true_type{});
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
    cu += G;
    if (cu >= U) break;  // (the loads issued after the last block are drained below)
    C = unit_of<BM, BN>(cu, tiles_m, tiles_n, nsplit, nkb);
    ckb = C.kb0;
  }
  // no direct-to-LDS load may still be writing when the workgroup's LDS is handed to the next one
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Sum of the split partial sums in split order, converted to the output type:
// out[m, n] = sum_s partial[s][m][n]  (OUTF32 == 2: out[m, n] += that sum, in FP32).
template <int OUTF32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int nsplit, int64_t M,
                                                            int64_t N, void* __restrict__ out, int64_t ldo) {
  const int64_t total = M * (N / 4);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / (N / 4), n = 4 * (i - m * (N / 4));
    v4f s = *reinterpret_cast<const v4f*>(partial + m * N + n);
    for (int k = 1; k < nsplit; ++k) s += *reinterpret_cast<const v4f*>(partial + ((int64_t)k * M + m) * N + n);
    if constexpr (OUTF32 == 2) {
      v4f* o = reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + m * ldo + n);
      *o = *o + s;
    } else if constexpr (OUTF32) {
      *reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + m * ldo + n) = s;
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + m * ldo + n) =
          make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
    }
  }
}

template <int OP, int BM, int BN, int WGM, int WGN, int NSTAGE, int SBM, int FA, int FB, int OUTF32>
static hipError_t launch_variant(const GemmDesc& d, const GemmPlan& p, float* partial, hipStream_t st) {
  hipLaunchKernelGGL((gemm_tn_kernel<OP, BM, BN, WGM, WGN, NSTAGE, SBM, FA, FB, OUTF32>), dim3((unsigned)p.grid),
                     dim3(WGM * WGN * 64), 0, st, d, (uint32_t)p.tiles_m, (uint32_t)p.tiles_n, p.split_k, partial);
  return hipGetLastError();
}

template <int OP, int SBM, int FA, int FB, int OUTF32>
static hipError_t launch_fmt(const GemmDesc& d, const GemmPlan& p, float* partial, hipStream_t st) {
  switch (p.shape) {
    case k128x256: return launch_variant<OP, 128, 256, 2, 4, 2, SBM, FA, FB, OUTF32>(d, p, partial, st);
    case k256x128: return launch_variant<OP, 256, 128, 4, 2, 2, SBM, FA, FB, OUTF32>(d, p, partial, st);
    case k256x256: return launch_variant<OP, 256, 256, 2, 4, 2, SBM, FA, FB, OUTF32>(d, p, partial, st);
    case k64x64: return launch_variant<OP, 64, 64, 4, 1, 2, SBM, FA, FB, OUTF32>(d, p, partial, st);
    default: return launch_variant<OP, 128, 128, 2, 2, 2, SBM, FA, FB, OUTF32>(d, p, partial, st);
  }
}

template <int OP, int SBM, int OUTF32>
static hipError_t launch_formats(const GemmDesc& d, const GemmPlan& p, float* partial, hipStream_t st) {
  if (d.fa == kE4M3 && d.fb == kE4M3) return launch_fmt<OP, SBM, kE4M3, kE4M3, OUTF32>(d, p, partial, st);
  if (d.fa == kE5M2 && d.fb == kE4M3) return launch_fmt<OP, SBM, kE5M2, kE4M3, OUTF32>(d, p, partial, st);
  if (d.fa == kE4M3 && d.fb == kE5M2) return launch_fmt<OP, SBM, kE4M3, kE5M2, OUTF32>(d, p, partial, st);
  return launch_fmt<OP, SBM, kE5M2, kE5M2, OUTF32>(d, p, partial, st);
}

template <int OP, int SBM>
static hipError_t launch_out(const GemmDesc& d, const GemmPlan& p, float* partial, hipStream_t st) {
  if constexpr (OP == kOpWgrad) {
    if (d.out_f32 == 2) return launch_formats<OP, SBM, 2>(d, p, partial, st);
  }
  return d.out_f32 ? launch_formats<OP, SBM, 1>(d, p, partial, st) : launch_formats<OP, SBM, 0>(d, p, partial, st);
}

hipError_t launch_gemm(int op, const GemmDesc& d, const GemmPlan& p, void* ws, hipStream_t st) {
  float* partial = p.split_k > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  hipError_t e;
  if (op == kOpFprop)
    e = launch_out<kOpFprop, kSbBlock128>(d, p, partial, st);
  else if (op == kOpDgrad)
    e = launch_out<kOpDgrad, kSbBlock128>(d, p, partial, st);
  else
    e = launch_out<kOpWgrad, kSbColumn>(d, p, partial, st);
  if (e != hipSuccess || p.split_k <= 1) return e;
  const int64_t total = d.M * (d.N / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (d.out_f32 == 2)
    hipLaunchKernelGGL(splitk_reduce_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, partial, p.split_k, d.M,
                       d.N, d.c, d.ldc);
  else if (d.out_f32)
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, partial, p.split_k, d.M,
                       d.N, d.c, d.ldc);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, partial, p.split_k, d.M,
                       d.N, d.c, d.ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Byte transpose, 128x128 tiles: each thread loads a 4-row x 16-byte patch, transposes 4x4 byte
// blocks with v_perm_b32, stages dwords (4 source rows of one column) in LDS, and writes 16-byte
// runs of the destination rows.
// ---------------------------------------------------------------------------------------------
constexpr int kTrStride = 33;

__device__ __forceinline__ void transpose4x4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, uint32_t (&o)[4]) {
  // v_perm_b32(hi, lo, sel): byte i of the result is byte sel_i of the 8-byte value {hi, lo}.
  const uint32_t p01l = __builtin_amdgcn_perm(d1, d0, 0x05010400u);  // d0.b0 d1.b0 d0.b1 d1.b1
  const uint32_t p01h = __builtin_amdgcn_perm(d1, d0, 0x07030602u);  // d0.b2 d1.b2 d0.b3 d1.b3
  const uint32_t p23l = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
  const uint32_t p23h = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);  // d0.b0 d1.b0 d2.b0 d3.b0
  o[1] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
}

__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ src, int64_t lds,
                                                           uint8_t* __restrict__ dst, int64_t ldd, uint32_t ncb) {
  __shared__ uint32_t tileT[128 * kTrStride];
  const int t = threadIdx.x;
  const TileRC tile = tile_of_block(ncb);
  const int64_t r0 = tile.row * 128, c0 = tile.col * 128;
  const int rq = t >> 3, cq = t & 7;
  uint4 d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) d[p] = *reinterpret_cast<const uint4*>(src + (r0 + 4 * rq + p) * lds + c0 + 16 * cq);
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&d[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&d[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&d[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&d[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t o[4];
    transpose4x4(w0[w], w1[w], w2[w], w3[w], o);
#pragma unroll
    for (int b = 0; b < 4; ++b) tileT[(16 * cq + 4 * w + b) * kTrStride + rq] = o[b];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int id = t + 256 * pass, k = id >> 3, ch = id & 7;
    const uint32_t* s4 = tileT + k * kTrStride + 4 * ch;
    *reinterpret_cast<uint4*>(dst + (c0 + k) * ldd + r0 + 16 * ch) = make_uint4(s4[0], s4[1], s4[2], s4[3]);
  }
}

hipError_t launch_transpose_u8(const uint8_t* src, int64_t lds, uint8_t* dst, int64_t ldd, int64_t R, int64_t C,
                               hipStream_t st) {
  const uint32_t ncb = (uint32_t)(C / 128);
  hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)(R / 128) * ncb), dim3(256), 0, st, src, lds, dst, ldd, ncb);
  return hipGetLastError();
}

__global__ void zero_fill_kernel(uint8_t* dst, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
  const int64_t total = rows * row_bytes;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / row_bytes, c = i - r * row_bytes;
    dst[r * ld_bytes + c] = 0;
  }
}

hipError_t launch_zero_fill(void* dst, int64_t rows, int64_t row_bytes, int64_t ld_bytes, hipStream_t st) {
  const int64_t total = rows * row_bytes;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint8_t*)dst, rows, row_bytes,
                     ld_bytes);
  return hipGetLastError();
}

}  // namespace fp8bq
