// Helpers shared by the MFMA kernels: direct global->LDS loads, their waits,
// the XOR swizzle of LDS tiles, and the accumulator layout of the 32x32 MFMA.
//
//   * A direct global->LDS load (global_load_lds_dwordx4) moves 16 bytes per
//     lane, 1 KB per wave instruction = 8 rows x 128 bytes of a tile with
//     64-wide K blocks: whole 128-byte lines, no registers.
//   * Inside an LDS block the eight 16-byte chunks of a row are XOR-swizzled
//     by row (chunk c of row r sits at slot c ^ g(r), g(r) = (r ^ (r >> 3))
//     mod 8), so a ds_read_b128 of 16 consecutive rows touches 16 distinct
//     slots of a 256-byte bank window (and 8 consecutive rows 8 distinct slots
//     of a 128-byte one): conflict-free.  The swizzle is applied by choosing
//     each lane's global source address.
//   * Waits are explicit (s_waitcnt vmcnt), followed by a plain s_barrier: a
//     fenced barrier would drain every load in flight.
//   * The K mapping is the same permutation for both operands (chunk 2i +
//     lane/32 of a 64-wide block feeds MFMA step i), so the products are those
//     of plain row-major operands.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kPipeBK = 64;          // K per LDS block
constexpr int kPipeThreads = 256;    // 4 waves

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// LDS byte address lds_base + 16 l.  Issued through inline asm so that the
// compiler does not see an LDS write it cannot place relative to the reads of
// the other stages (it would drain every load before each read); the waits
// are explicit instead.  The instruction has no register results.
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

// Row of register r of a 32x32 MFMA accumulator for this lane (the column is
// lane & 31).
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace moe
