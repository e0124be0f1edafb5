// Main loop of the grouped GEMMs: weights streamed from HBM straight into MFMA
// registers, token rows staged in LDS.
//
// A workgroup of 4 waves computes, for BM token rows and 256 weight rows,
// C^T[256 x BM] = W[256 x K] * A[BM x K]^T with v_mfma_f32_32x32x16_bf16 (fp32
// accumulation).  Wave w owns two 32-row weight blocks and all BM token rows.
//   * Weights are stored packed in MFMA fragment order (moe_pack_weights): the
//     operand of one wave for one 32-row block and one 16-wide K step is 1 KB
//     of contiguous memory, lane l holding 16 bytes.  Each wave streams its two
//     blocks with whole-line 16-byte loads into a ring of PF steps of registers
//     -- register space is far larger than LDS, so many bytes are in flight per
//     CU, which is what an HBM-bound stream needs.
//   * Token rows (gathered through the expert order, L2/MALL resident) move by
//     direct global->LDS loads (global_load_lds_dwordx4) into a ring of NS
//     stages of 64-wide K blocks, 32-row groups past the tile's rows not
//     loaded; chunks XOR-swizzled by row for conflict-free ds_read_b128.
//   * The LDS loads are issued through inline asm (the compiler cannot place
//     them against the reads of other stages and would drain every load), so
//     their waits are explicit; the register loads are ordinary loads whose
//     waits the compiler derives.
//   * Token blocks past the tile's valid rows skip their MFMAs (a compile-time
//     count per specialisation).
// The weight operand is the MFMA's first operand: in an accumulator lane l holds
// token (l mod 32) of its block and register quad q four consecutive weight
// rows, so epilogues store four adjacent outputs of one token at once.
#pragma once

#include <type_traits>

#include "mma_pipeline.h"

namespace moe {

constexpr int kStreamBK = 64;        // K per LDS stage (4 MFMA steps)
constexpr int kStreamRows = 256;     // weight rows per tile (4 waves x 2 blocks)

template <int BM>
struct StreamTile {
  static constexpr int MBW = BM / 32;             // token blocks (every wave covers all)
  // weight steps in flight per wave (two 16-byte registers quads each), as
  // many as the registers left beside BM / 32 x 2 accumulator tiles allow
  static constexpr int PF = BM >= 192 ? 12 : 16;
  static constexpr int kAElems = BM * kStreamBK;  // one LDS stage
  static constexpr int kAGroups = BM / 32;        // 32-row load groups (one instruction per wave)
};

// LDS chunk slot of lane `lane` in A group g of wave `wave`: the four waves'
// instructions of group g cover token rows [32 g, 32 g + 32), 8 rows each.
__device__ __forceinline__ int stream_a_slot(int g, int wave, int lane) {
  return (g * 4 + wave) * 64 + lane;
}

// Ring for MBV valid token blocks (1..MBW); the MBV 32-row groups that hold
// them are the ones loaded per stage.  a_src[g]: this lane's token-row source
// for group g at K = 0; wsrc[j]: this lane's packed-weight source for block j
// at step 0.
template <int BM, int NS, int MBV>
__device__ __forceinline__ void stream_ring(const bf16_t* const* a_src, const bf16_t* const* wsrc,
                                            int NKB, bf16_t* lds, f32x16 (&acc)[StreamTile<BM>::MBW][2]) {
  using ST = StreamTile<BM>;
  constexpr int PF = ST::PF;
  constexpr int U = PF / 4;                            // K blocks per unrolled loop body
  static_assert(PF % 4 == 0 && U >= 1 && U <= 4, "prefetch ring");
  constexpr uint32_t kStageBytes = ST::kAElems * 2;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int NKS = NKB * 4;
  // loads issued after a stage's LDS loads, up to the wait before its use: the
  // weight loads of NS - 1 blocks (8 each) and the LDS loads of NS - 2 stages
  constexpr int keep = 8 * (NS - 1) + (NS - 2) * MBV;
  static_assert(MBV >= 1 && keep < 64, "wait count");

  const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_addr(lds + (stream_a_slot(0, wave, 0) << 3)));
  auto issue = [&](int st, int kb) {
    const uint32_t off = static_cast<uint32_t>(st) * kStageBytes;
#pragma unroll
    for (int g = 0; g < ST::kAGroups; ++g)
      if (g < MBV) dma16(a_src[g] + kb * kStreamBK, a_dst + off + g * 4096);
  };

  u32x4 bq[PF][2];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, NKB - 1));
  // issued in step order: the compiler derives the wait before each step's
  // MFMAs from the order it sees on entry to the loop, so an out-of-order
  // prologue would make it wait for every load at the top of each iteration
#pragma unroll
  for (int p = 0; p < PF; ++p) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bq[p][j] = *reinterpret_cast<const u32x4*>(wsrc[j] + static_cast<size_t>(min(p, NKS - 1)) * 512);
    __builtin_amdgcn_sched_barrier(0);
  }

  int st = 0;                                          // kb % NS
  // one K block; u: its position in the unrolled body (ring slots 4u..4u+3)
  auto kblock = [&](int kb, auto u_tag) {
    constexpr int u = decltype(u_tag)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_only(keep));
    __builtin_amdgcn_s_barrier();
    issue(st == 0 ? NS - 1 : st - 1, min(kb + NS - 1, NKB - 1));
    const bf16_t* As = lds + st * ST::kAElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      constexpr int sl0 = u * 4;                       // == 4 kb % PF
      const int ch = 2 * i + (lane >> 5);
      bf16x8 fa[MBV];
#pragma unroll
      for (int m = 0; m < MBV; ++m)
        fa[m] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&As[pipe_swz(32 * m + (lane & 31), ch)]));
      const bf16x8 w0 = __builtin_bit_cast(bf16x8, bq[sl0 + i][0]);
      const bf16x8 w1 = __builtin_bit_cast(bf16x8, bq[sl0 + i][1]);
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, fa[m], acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, fa[m], acc[m][1], 0, 0, 0);
      }
      const size_t nxt = static_cast<size_t>(min(4 * kb + i + PF, NKS - 1)) * 512;
#pragma unroll
      for (int j = 0; j < 2; ++j) bq[sl0 + i][j] = *reinterpret_cast<const u32x4*>(wsrc[j] + nxt);
      // keep each refill right after the step that frees its registers: the
      // scheduler would otherwise sink the loads and shorten the prefetch
      __builtin_amdgcn_sched_barrier(0);
    }
    st = st + 1 == NS ? 0 : st + 1;
  };
  int kb0 = 0;
  for (; kb0 + U <= NKB; kb0 += U) {
    kblock(kb0, std::integral_constant<int, 0>{});
    if constexpr (U > 1) kblock(kb0 + 1, std::integral_constant<int, 1>{});
    if constexpr (U > 2) kblock(kb0 + 2, std::integral_constant<int, 2>{});
    if constexpr (U > 3) kblock(kb0 + 3, std::integral_constant<int, 3>{});
  }
  // remaining K blocks (NKB mod U)
  if constexpr (U > 1) {
    if (kb0 < NKB) kblock(kb0, std::integral_constant<int, 0>{});
    if constexpr (U > 2) {
      if (kb0 + 1 < NKB) kblock(kb0 + 1, std::integral_constant<int, 1>{});
      if constexpr (U > 3)
        if (kb0 + 2 < NKB) kblock(kb0 + 2, std::integral_constant<int, 2>{});
    }
  }
  // drain the tail loads (clamped, unused) before the caller reuses registers
  // and LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __builtin_amdgcn_s_barrier();
}

// NKB = K / 64, a multiple of kStreamPF / 4.  valid_rows: token rows of the
// tile that hold data (1..BM).  epi(acc) runs once per specialisation after the
// ring (every load landed, every wave past a barrier after its last LDS read);
// acc[m][j]: lane l is token 32 m + (l mod 32), register r is weight row
// (block j) + mfma32_row(r, l).
template <int BM, int NS, typename Epi>
__device__ __forceinline__ void stream_pipeline(const bf16_t* const* a_src, const bf16_t* const* wsrc,
                                                int NKB, int valid_rows, bf16_t* lds, Epi&& epi) {
  using ST = StreamTile<BM>;
  auto run = [&](auto mbv_tag) {
    constexpr int MBV = decltype(mbv_tag)::value;
    f32x16 acc[ST::MBW][2];
#pragma unroll
    for (int m = 0; m < ST::MBW; ++m) {
      acc[m][0] = f32x16{0.f};
      acc[m][1] = f32x16{0.f};
    }
    stream_ring<BM, NS, MBV>(a_src, wsrc, NKB, lds, acc);
    epi(acc);
  };
  // all waves cover all token rows, so the count is uniform
  const int mbv = min(ST::MBW, (valid_rows + 31) >> 5);
  static_assert(ST::MBW <= 8, "token blocks");
  switch (mbv) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (ST::MBW >= 2) run(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (ST::MBW >= 3) run(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (ST::MBW >= 4) run(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr (ST::MBW >= 5) run(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr (ST::MBW >= 6) run(std::integral_constant<int, 6>{}); break;
    case 7: if constexpr (ST::MBW >= 7) run(std::integral_constant<int, 7>{}); break;
    default: run(std::integral_constant<int, ST::MBW>{}); break;
  }
}

}  // namespace moe
