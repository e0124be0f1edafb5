// Pipelined bf16 MFMA main loop shared by the router and the grouped GEMMs.
//
// A workgroup of 4 waves computes C[BM x 256] += A[BM x K] * B[256 x K]^T with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).
//   * Both operands stream into LDS with direct global->LDS loads
//     (global_load_lds_dwordx4): each wave instruction moves 1 KB = 8 rows x
//     128 bytes, so every load uses whole 128-byte lines and needs no
//     registers.  NS stages of 64-wide K blocks form a ring; NS - 1 of them are
//     in flight while one is consumed.
//   * Inside a stage, the 16-byte chunks of a row are XOR-swizzled by row
//     (chunk c of row r sits at slot c ^ g(r), g(r) = (r ^ r/8) mod 8), so a
//     ds_read_b128 of 16 consecutive rows touches 16 distinct 16-byte slots of
//     a 256-byte bank window (and 8 consecutive rows 8 distinct slots of a
//     128-byte one): conflict-free.  The swizzle is applied by choosing each
//     lane's global source address.
//   * Waits are explicit: before consuming stage kb every wave waits until at
//     most (NS - 2) stages of its own loads are outstanding, then the workgroup
//     meets at a plain s_barrier (a fenced barrier would drain every load).
//   * Wave w multiplies all BM rows of A by its two 32-row blocks of B
//     (bq_row[0], bq_row[1] inside the 256-row B tile); 32-row blocks at or
//     past `mb_valid` skip their MFMAs.
// The K mapping is the same permutation for A and B (chunk 2i + lane/32 of a
// 64-wide block feeds step i), so the products are those of plain row-major
// operands.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kPipeBK = 64;          // K per stage
constexpr int kPipeThreads = 256;    // 4 waves
constexpr int kPipeBRows = 256;      // B rows per tile

typedef __attribute__((address_space(3))) void lds_void_t;

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

__device__ __forceinline__ int swz_key(int row) { return (row ^ (row >> 3)) & 7; }

// element offset of 16-byte chunk `ch` of row `row` in a [rows][64] bf16 tile
__device__ __forceinline__ int pipe_swz(int row, int ch) {
  return row * kPipeBK + ((ch ^ swz_key(row)) << 3);
}

template <int BM, int NS>
struct PipeShape {
  static constexpr int kAElems = BM * kPipeBK;
  static constexpr int kBElems = kPipeBRows * kPipeBK;
  static constexpr int kStageElems = kAElems + kBElems;
  static constexpr int kLdsElems = NS * kStageElems;
  static constexpr int kAInst = BM / 32;        // A DMA instructions per wave per stage
  static constexpr int kBInst = 8;              // B DMA instructions per wave per stage
  static constexpr int kInst = kAInst + kBInst;
};

// Global source, at K = 0, of the chunk this lane moves in DMA instruction q of
// its wave for a tile of `rows` rows: the chunk that the swizzle places at the
// lane's LDS slot.  Returns (row, element offset inside the row).
template <int INST_PER_WAVE>
__device__ __forceinline__ void dma_chunk(int q, int& row, int& col) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = (wave * INST_PER_WAVE + q) * 64 + lane;
  row = P >> 3;
  col = ((P & 7) ^ swz_key(row)) << 3;
}

// MFMA operand fragments of one 16-wide K step: MBV A blocks and 2 B blocks.
template <int MBV>
struct StepFrags {
  bf16x8 a[MBV];
  bf16x8 b[2];
};

template <int MBV>
__device__ __forceinline__ void load_frags(StepFrags<MBV>& f, const bf16_t* As, const bf16_t* Bs,
                                           const int (&brow)[2], int i, int lane) {
  const int ch = 2 * i + (lane >> 5);
#pragma unroll
  for (int m = 0; m < MBV; ++m)
    f.a[m] = __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const u32x4*>(&As[pipe_swz(32 * m + (lane & 31), ch)]));
#pragma unroll
  for (int j = 0; j < 2; ++j)
    f.b[j] = __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const u32x4*>(&Bs[pipe_swz(brow[j] + (lane & 31), ch)]));
}

// The ring for a tile whose first MBV 32-row blocks hold rows (MBV <= BM/32):
// one loop without branches, the MFMA count fixed at compile time, and the
// fragments of step i+1 read from LDS while the MFMAs of step i issue.
template <int BM, int NS, int MBV>
__device__ __forceinline__ void mma_ring(const bf16_t* const* a_src, const bf16_t* const* b_src,
                                         int NKB, const int (&brow)[2], bf16_t* lds,
                                         f32x16 (&acc)[BM / 32][2]) {
  using PS = PipeShape<BM, NS>;
  static_assert(NS >= 2 && (NS - 2) * PS::kInst < 64, "vmcnt range");
  constexpr uint32_t kStageBytes = PS::kStageElems * 2;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  // wave-uniform LDS byte addresses of this wave's first A and B slots in stage 0
  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_addr(lds + wave * PS::kAInst * 512));
  const uint32_t b_dst =
      __builtin_amdgcn_readfirstlane(lds_addr(lds + PS::kAElems + wave * PS::kBInst * 512));
  auto issue = [&](int st, int kb) {
    const uint32_t off = static_cast<uint32_t>(st) * kStageBytes;
#pragma unroll
    for (int q = 0; q < PS::kAInst; ++q) dma16(a_src[q] + kb * kPipeBK, a_dst + off + q * 1024);
#pragma unroll
    for (int q = 0; q < PS::kBInst; ++q) dma16(b_src[q] + kb * kPipeBK, b_dst + off + q * 1024);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, NKB - 1));

  int st = 0;                                          // kb % NS
  for (int kb = 0; kb < NKB; ++kb) {
    __builtin_amdgcn_s_waitcnt(vmcnt_only((NS - 2) * PS::kInst));
    __builtin_amdgcn_s_barrier();
    // refill the stage consumed in the previous step (every wave is past it)
    issue(st == 0 ? NS - 1 : st - 1, min(kb + NS - 1, NKB - 1));
    const bf16_t* As = lds + st * PS::kStageElems;
    const bf16_t* Bs = As + PS::kAElems;
    StepFrags<MBV> f[2];
    load_frags<MBV>(f[0], As, Bs, brow, 0, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 1 < 4) load_frags<MBV>(f[(i + 1) & 1], As, Bs, brow, i + 1, lane);
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i & 1].a[m], f[i & 1].b[0], acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i & 1].a[m], f[i & 1].b[1], acc[m][1], 0, 0, 0);
      }
    }
    st = st + 1 == NS ? 0 : st + 1;
  }
  // the tail refills (clamped, unused) may still be landing: drain before the
  // caller reuses the LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __builtin_amdgcn_s_barrier();
}

// a_src[q], b_src[q]: this lane's DMA sources at K = 0 (see dma_chunk).
// lds: NS * PipeShape::kStageElems bf16 elements.
// NKB = K / 64 (any value >= 1).  Blocks at or past mb_valid are left at zero.
// On return all loads have landed and every wave has passed a barrier after
// its last LDS read.
template <int BM, int NS>
__device__ __forceinline__ void mma_pipeline(const bf16_t* const* a_src, const bf16_t* const* b_src,
                                             int NKB, int mb_valid, const int (&brow)[2],
                                             bf16_t* lds, f32x16 (&acc)[BM / 32][2]) {
  constexpr int MB = BM / 32;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    acc[m][0] = f32x16{0.f};
    acc[m][1] = f32x16{0.f};
  }
  if (mb_valid >= MB || MB == 1) {
    mma_ring<BM, NS, MB>(a_src, b_src, NKB, brow, lds, acc);
  } else if constexpr (MB >= 2) {
    if (mb_valid == 1) mma_ring<BM, NS, 1>(a_src, b_src, NKB, brow, lds, acc);
    else if constexpr (MB >= 3) {
      if (mb_valid == 2) mma_ring<BM, NS, 2>(a_src, b_src, NKB, brow, lds, acc);
      else if constexpr (MB >= 4) mma_ring<BM, NS, 3>(a_src, b_src, NKB, brow, lds, acc);
    }
  }
}

// Row of register r of a 32x32 MFMA accumulator for this lane (the column is
// lane & 31).
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace moe
