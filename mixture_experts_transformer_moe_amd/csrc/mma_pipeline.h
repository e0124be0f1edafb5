// Pipelined bf16 MFMA main loop shared by the router and the grouped GEMMs.
//
// A workgroup of 4 waves computes, for a tile of BM "A" rows (tokens) and BN
// "B" rows (weight rows), C^T[BN x BM] = B[BN x K] * A[BM x K]^T with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  The weight block is the MFMA's
// first operand, so in an accumulator lane l holds token (l mod 32) and four
// consecutive weight rows per register quad: epilogues store 4 adjacent outputs
// of one token straight from registers.
//   * Both operands stream into LDS with direct global->LDS loads
//     (global_load_lds_dwordx4): a wave instruction moves 1 KB = 8 rows x 128
//     bytes, whole 128-byte lines, and needs no registers.  NS stages of
//     64-wide K blocks form a ring; NS - 1 of them are in flight while one is
//     consumed.
//   * A rows are loaded in groups of 32 (one instruction per wave per group);
//     groups past the tile's valid rows are not loaded at all.
//   * Inside a stage the eight 16-byte chunks of a row are XOR-swizzled by row
//     (chunk c of row r sits at slot c ^ g(r), g(r) = (r ^ (r >> 3)) mod 8), so
//     a ds_read_b128 of 16 consecutive rows touches 16 distinct slots of a
//     256-byte bank window (and 8 consecutive rows 8 distinct slots of a
//     128-byte one): conflict-free.  The swizzle is applied by choosing each
//     lane's global source address.
//   * Waits are explicit: before consuming stage kb every wave waits until at
//     most (NS - 2) stages of its own loads are outstanding, then the workgroup
//     meets at a plain s_barrier (a fenced barrier would drain every load).
//   * Waves form a WM x WN grid: wave (wm, wn) multiplies the tile's token rows
//     [wm RW, wm RW + RW) by two 32-row weight blocks listed in brow[]; token
//     blocks past the valid rows skip their MFMAs (a compile-time count per
//     specialisation).
// The K mapping is the same permutation for both operands (chunk 2i + lane/32
// of a 64-wide block feeds step i), so the products are those of plain
// row-major operands.
#pragma once

#include <type_traits>

#include "moe_internal.h"

namespace moe {

constexpr int kPipeBK = 64;          // K per stage
constexpr int kPipeThreads = 256;    // 4 waves

template <int BM, int BN>
struct PipeTile {
  static constexpr int WM = BM >= 64 ? 2 : 1;     // waves along tokens
  static constexpr int WN = 4 / WM;               // waves along weight rows
  static constexpr int RW = BM / WM;              // token rows per wave
  static constexpr int MBW = RW / 32;             // 32-token blocks per wave
  static constexpr int NBW = BN / 32 / WN;        // 32-row weight blocks per wave
  static constexpr int kAElems = BM * kPipeBK;
  static constexpr int kBElems = BN * kPipeBK;
  static constexpr int kStageElems = kAElems + kBElems;
  static constexpr int kAGroups = BM / 32;        // A load groups (one instruction per wave each)
  static constexpr int kBInst = BN / 32;          // B DMA instructions per wave per stage
  static_assert(RW % 32 == 0 && NBW == 2, "tile shape");
};

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// LDS byte address lds_base + 16 l.  Issued through inline asm so that the
// compiler does not see an LDS write it cannot place relative to the reads of
// the other stages (it would drain every load before each read); the ring's
// waits are explicit instead.  The instruction has no register results.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding).
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// s_waitcnt vmcnt(n) for a run-time n in [0, 64) (out of range: wait for all).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define MOE_VMCNT_CASE(v) \
  case v:                 \
    __builtin_amdgcn_s_waitcnt(vmcnt_only(v)); \
    break;
  switch (n) {
    MOE_VMCNT_CASE(0) MOE_VMCNT_CASE(1) MOE_VMCNT_CASE(2) MOE_VMCNT_CASE(3) MOE_VMCNT_CASE(4)
    MOE_VMCNT_CASE(5) MOE_VMCNT_CASE(6) MOE_VMCNT_CASE(7) MOE_VMCNT_CASE(8) MOE_VMCNT_CASE(9)
    MOE_VMCNT_CASE(10) MOE_VMCNT_CASE(11) MOE_VMCNT_CASE(12) MOE_VMCNT_CASE(13) MOE_VMCNT_CASE(14)
    MOE_VMCNT_CASE(15) MOE_VMCNT_CASE(16) MOE_VMCNT_CASE(17) MOE_VMCNT_CASE(18) MOE_VMCNT_CASE(19)
    MOE_VMCNT_CASE(20) MOE_VMCNT_CASE(21) MOE_VMCNT_CASE(22) MOE_VMCNT_CASE(23) MOE_VMCNT_CASE(24)
    MOE_VMCNT_CASE(25) MOE_VMCNT_CASE(26) MOE_VMCNT_CASE(27) MOE_VMCNT_CASE(28) MOE_VMCNT_CASE(29)
    MOE_VMCNT_CASE(30) MOE_VMCNT_CASE(31) MOE_VMCNT_CASE(32) MOE_VMCNT_CASE(33) MOE_VMCNT_CASE(34)
    MOE_VMCNT_CASE(35) MOE_VMCNT_CASE(36) MOE_VMCNT_CASE(37) MOE_VMCNT_CASE(38) MOE_VMCNT_CASE(39)
    MOE_VMCNT_CASE(40) MOE_VMCNT_CASE(41) MOE_VMCNT_CASE(42) MOE_VMCNT_CASE(43) MOE_VMCNT_CASE(44)
    MOE_VMCNT_CASE(45) MOE_VMCNT_CASE(46) MOE_VMCNT_CASE(47) MOE_VMCNT_CASE(48) MOE_VMCNT_CASE(49)
    MOE_VMCNT_CASE(50) MOE_VMCNT_CASE(51) MOE_VMCNT_CASE(52) MOE_VMCNT_CASE(53) MOE_VMCNT_CASE(54)
    MOE_VMCNT_CASE(55) MOE_VMCNT_CASE(56) MOE_VMCNT_CASE(57) MOE_VMCNT_CASE(58) MOE_VMCNT_CASE(59)
    MOE_VMCNT_CASE(60) MOE_VMCNT_CASE(61) MOE_VMCNT_CASE(62) MOE_VMCNT_CASE(63)
    default: __builtin_amdgcn_s_waitcnt(vmcnt_only(0)); break;
  }
#undef MOE_VMCNT_CASE
}

__device__ __forceinline__ int swz_key(int row) { return (row ^ (row >> 3)) & 7; }

// element offset of 16-byte chunk `ch` (0..7) of row `row` in a [rows][64] bf16 tile
__device__ __forceinline__ int pipe_swz(int row, int ch) {
  return row * kPipeBK + ((ch ^ swz_key(row)) << 3);
}

// Global source (row, element offset in the row) of the bytes that land in LDS
// chunk slot P (16 bytes each, 8 per row) under the swizzle.
__device__ __forceinline__ void chunk_source(int P, int& row, int& col) {
  row = P >> 3;
  col = ((P & 7) ^ swz_key(row)) << 3;
}

// LDS chunk slot of lane `lane` in A group g of wave `wave`: the four waves'
// instructions of group g cover token rows [32 g, 32 g + 32), 8 rows each.
__device__ __forceinline__ int a_slot(int g, int wave, int lane) { return (g * 4 + wave) * 64 + lane; }

template <int BN>
__device__ __forceinline__ int b_slot(int q, int wave, int lane) { return (wave * (BN / 32) + q) * 64 + lane; }

// DMA sources of this lane at K = 0, for a tile whose token rows start at
// a_row(r) and weight rows at b_row(r).
template <int BM, int BN, typename ARow, typename BRow>
__device__ __forceinline__ void pipe_sources(const bf16_t** a_src, const bf16_t** b_src, ARow a_row,
                                             BRow b_row) {
  using PT = PipeTile<BM, BN>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int g = 0; g < PT::kAGroups; ++g) {
    int row, col;
    chunk_source(a_slot(g, wave, lane), row, col);
    a_src[g] = a_row(row) + col;
  }
#pragma unroll
  for (int q = 0; q < PT::kBInst; ++q) {
    int row, col;
    chunk_source(b_slot<BN>(q, wave, lane), row, col);
    b_src[q] = b_row(row) + col;
  }
}

// The ring for a wave whose first MBV token blocks hold rows; `groups` A load
// groups (tile-wide, >= 1) are loaded per stage.  No branches around the loads
// inside the loop, the MFMA count fixed at compile time.
template <int BM, int BN, int NS, int MBV>
__device__ __forceinline__ void mma_ring(const bf16_t* const* a_src, const bf16_t* const* b_src,
                                         int NKB, int groups, const int (&brow)[2], bf16_t* lds,
                                         f32x16 (&acc)[PipeTile<BM, BN>::MBW][2]) {
  using PT = PipeTile<BM, BN>;
  constexpr uint32_t kStageBytes = PT::kStageElems * 2;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int arow0 = (wave / PT::WN) * PT::RW;
  const int per_stage = groups + PT::kBInst;                 // loads per wave per stage
  const int keep = (NS - 2) * per_stage;                     // may stay in flight

  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_addr(lds + (a_slot(0, wave, 0) << 3)));
  const uint32_t b_dst =
      __builtin_amdgcn_readfirstlane(lds_addr(lds + PT::kAElems + (b_slot<BN>(0, wave, 0) << 3)));
  auto issue = [&](int st, int kb) {
    const uint32_t off = static_cast<uint32_t>(st) * kStageBytes;
#pragma unroll
    for (int g = 0; g < PT::kAGroups; ++g)
      if (g < groups) dma16(a_src[g] + kb * kPipeBK, a_dst + off + g * 4096);
#pragma unroll
    for (int q = 0; q < PT::kBInst; ++q) dma16(b_src[q] + kb * kPipeBK, b_dst + off + q * 1024);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, NKB - 1));

  int st = 0;                                          // kb % NS
  for (int kb = 0; kb < NKB; ++kb) {
    wait_vmcnt(keep);
    __builtin_amdgcn_s_barrier();
    // refill the stage consumed in the previous step (every wave is past it)
    issue(st == 0 ? NS - 1 : st - 1, min(kb + NS - 1, NKB - 1));
    if constexpr (MBV > 0) {
      const bf16_t* As = lds + st * PT::kStageElems;
      const bf16_t* Bs = As + PT::kAElems;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 2 * i + (lane >> 5);
        bf16x8 fa[MBV], fb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[j] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&Bs[pipe_swz(brow[j] + (lane & 31), ch)]));
#pragma unroll
        for (int m = 0; m < MBV; ++m)
          fa[m] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&As[pipe_swz(arow0 + 32 * m + (lane & 31), ch)]));
#pragma unroll
        for (int m = 0; m < MBV; ++m)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[m], acc[m][j], 0, 0, 0);
      }
    }
    st = st + 1 == NS ? 0 : st + 1;
  }
  // the tail refills (clamped, unused) may still be landing: drain before the
  // caller reuses the LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __builtin_amdgcn_s_barrier();
}

// a_src[g], b_src[q]: this lane's DMA sources at K = 0 (pipe_sources).
// lds: NS * PipeTile::kStageElems bf16 elements.  NKB = K / 64 (>= 1).
// valid_rows: token rows of the tile that hold data (1..BM); token blocks past
// it are neither loaded nor multiplied, and their accumulators stay zero.
// epi(acc) runs after every load has landed and every wave has passed a
// barrier after its last LDS read; it is instantiated once per specialisation
// so that the accumulators never merge across them.  acc[m][j] holds C^T for
// token block m of the wave and weight block j: lane l is token 32 m + (l mod
// 32) of the wave's rows, register r is weight row brow[j] + mfma32_row(r, l).
template <int BM, int BN, int NS, typename Epi>
__device__ __forceinline__ void mma_pipeline(const bf16_t* const* a_src, const bf16_t* const* b_src,
                                             int NKB, int valid_rows, const int (&brow)[2],
                                             bf16_t* lds, Epi&& epi) {
  using PT = PipeTile<BM, BN>;
  const int groups = min(PT::kAGroups, (valid_rows + 31) >> 5);
  auto run = [&](auto mbv_tag) {
    constexpr int MBV = decltype(mbv_tag)::value;
    f32x16 acc[PT::MBW][2];
#pragma unroll
    for (int m = 0; m < PT::MBW; ++m) {
      acc[m][0] = f32x16{0.f};
      acc[m][1] = f32x16{0.f};
    }
    mma_ring<BM, BN, NS, MBV>(a_src, b_src, NKB, groups, brow, lds, acc);
    epi(acc);
  };
  const int wave = threadIdx.x >> 6;
  const int rows_here = valid_rows - (wave / PT::WN) * PT::RW;
  const int mbv = rows_here <= 0 ? 0 : min(PT::MBW, (rows_here + 31) >> 5);
  if (mbv >= PT::MBW) {
    run(std::integral_constant<int, PT::MBW>{});
  } else if (mbv == 0) {
    run(std::integral_constant<int, 0>{});
  } else if constexpr (PT::MBW >= 2) {
    if (mbv == 1) {
      run(std::integral_constant<int, 1>{});
    } else if constexpr (PT::MBW >= 3) {
      if (mbv == 2) run(std::integral_constant<int, 2>{});
      else if constexpr (PT::MBW >= 4) run(std::integral_constant<int, 3>{});
    }
  }
}

// Row of register r of a 32x32 MFMA accumulator for this lane (the column is
// lane & 31).
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace moe
