// Main loop of the grouped GEMMs: weights streamed from HBM straight into MFMA
// registers, token rows staged in LDS, one continuous stream across the tiles
// a persistent workgroup computes.
//
// A workgroup of 4 waves computes, for a tile of BM token rows and 256 weight
// rows, C^T[256 x BM] = W[256 x K] * A[BM x K]^T with v_mfma_f32_32x32x16_bf16
// (fp32 accumulation).  Wave w owns two 32-row weight blocks and all BM rows.
//   * Weights are stored packed in MFMA fragment order (moe_pack_weights): the
//     operand of one wave for one 32-row block and one 16-wide K step is 1 KB
//     of contiguous memory, lane l holding 16 bytes.  Each wave streams its two
//     blocks with whole-line 16-byte loads into a ring of PF steps of registers
//     -- register space is far larger than LDS, so many bytes are in flight per
//     CU, which is what an HBM-bound stream needs.
//   * Token rows (gathered through the expert order, L2/MALL resident) move by
//     direct global->LDS loads (global_load_lds_dwordx4) into a ring of NS
//     stages of 64-wide K blocks; chunks are XOR-swizzled by row for
//     conflict-free ds_read_b128.
//   * Neither ring drains between tiles: the last steps of a tile prefetch the
//     first weight steps and token-row blocks of the workgroup's next tile, so
//     the HBM stream of a workgroup only stops after its last tile.
//   * The LDS loads are issued through inline asm (the compiler cannot place
//     them against the reads of other stages and would drain every load), so
//     their waits are explicit and count exactly the loads issued after them;
//     the register loads are ordinary loads whose waits the compiler derives.
//   * Every tile loads and multiplies all BM rows (rows past its last one
//     repeat it and their results are dropped): the per-block load counts are
//     then the same for every tile, every wait is a constant, and one set of
//     registers holds the weight ring for all tiles.
// The weight operand is the MFMA's first operand: in an accumulator lane l holds
// token (l mod 32) of its block and register quad q four consecutive weight
// rows, so epilogues store four adjacent outputs of one token at once.
#pragma once

#include <type_traits>

#include "mma_pipeline.h"

namespace moe {

constexpr int kStreamBK = 64;        // K per LDS stage (4 MFMA steps)
constexpr int kStreamNS = 4;         // LDS stages
constexpr int kStreamPF = 16;        // weight steps in flight per wave
constexpr int kStreamKAlign = kStreamBK * kStreamPF / 4;   // every K is a multiple (256)

template <int BM>
struct StreamTile {
  static constexpr int MBW = BM / 32;             // token blocks (every wave covers all)
  static constexpr int kAElems = BM * kStreamBK;  // one LDS stage
};

// One 16-byte direct global->LDS load per lane from base + voff bytes; lane l's
// bytes land at LDS byte address lds_base + 16 l.  No register results.
// base and lds_base must be the same in every lane.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t voff, uint32_t lds_base) {
  // (readfirstlane returns int: widen each half as unsigned, or a low half
  // with bit 31 set would sign-extend over the high half)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const void*>(sb)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// LDS chunk slot (16 bytes, 8 per row) of lane `lane` in LDS load g of wave
// `wave`: each load fills 8 consecutive rows, and a wave's MBW loads cover the
// consecutive rows [8 MBW wave, 8 MBW (wave + 1)) of the tile.
template <int BM>
__device__ __forceinline__ int stream_a_slot(int g, int wave, int lane) {
  return (wave * StreamTile<BM>::MBW + g) * 64 + lane;
}

// Sources of one tile.  Everything but a_off is the same in every lane.
template <int BM>
struct StreamSrc {
  const bf16_t* a_base;                 // token rows: this lane's chunk of group g
  uint32_t a_off[StreamTile<BM>::MBW];  //   at K = 0 is at a_base + a_off[g] bytes
  const bf16_t* w[2];                   // the wave's two packed weight block rows
  int groups;                           // 32-row groups holding rows, 1..MBW (informational)
  int nkb;                              // K / 64, a multiple of kStreamPF / 4
};

// What stays in flight between tiles.
struct StreamState {
  u32x4 bq[kStreamPF][2];               // weight operands of the next PF steps
  int st;                               // LDS stage holding the next K block
};

// s_waitcnt vmcnt(kBase + n) for a run-time n in [0, kMax] (uniform).
template <int kMax, int kBase>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  static_assert(kBase + kMax < 64, "vmcnt range");
  if constexpr (kMax > 0) {
    if (n >= kMax) {
      __builtin_amdgcn_s_waitcnt(vmcnt_only(kBase + kMax));
      return;
    }
    wait_vmcnt_upto<kMax - 1, kBase>(n);
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kBase));
  }
}

// The LDS stage of K block kb: all MBW 32-row groups.
template <int BM>
__device__ __forceinline__ void stream_issue(const StreamSrc<BM>& s, int kb, uint32_t dst) {
  const bf16_t* base = s.a_base + kb * kStreamBK;
#pragma unroll
  for (int g = 0; g < StreamTile<BM>::MBW; ++g) dma16_off(base, s.a_off[g], dst + g * 1024);
}

template <int BM>
__device__ __forceinline__ uint32_t stream_stage_addr(const bf16_t* lds, int st) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return lds_addr(lds + st * StreamTile<BM>::kAElems + (stream_a_slot<BM>(0, wave, 0) << 3));
}

// Starts the stream with the first tile: its first NS - 1 token-row blocks,
// then its first PF weight steps in step order (the compiler derives the wait
// before each step from the order it sees on entry to the loop).
template <int BM>
__device__ __forceinline__ void stream_start(const StreamSrc<BM>& s, StreamState& ss, const bf16_t* lds) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int st = 0; st < kStreamNS - 1; ++st) stream_issue(s, st, stream_stage_addr<BM>(lds, st));
  ss.st = 0;
#pragma unroll
  for (int p = 0; p < kStreamPF; ++p) {
#pragma unroll
    for (int j = 0; j < 2; ++j) ss.bq[p][j] = *reinterpret_cast<const u32x4*>(s.w[j] + p * 512 + lane * 8);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Drains the stream after the last tile (its tail loads repeat the last step).
__device__ __forceinline__ void stream_finish() {
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

// One MFMA step for MBV valid token blocks: their A fragments from the LDS
// stage, then two MFMAs per block.
template <int MBV, int MBW>
__device__ __forceinline__ void stream_step(const bf16_t* As, int ch, const u32x4 (&bw)[2],
                                            f32x16 (&acc)[MBW][2]) {
  const int lane = threadIdx.x & 63;
  // pipe_swz(32 m + r, ch) = 2048 m + r * 64 + ((ch ^ swz_key(r) ^ 4 (m & 1)) << 3)
  // for r < 32: two lane offsets serve every block (the rest is an immediate)
  const int r = lane & 31;
  const int off0 = r * kStreamBK + ((ch ^ swz_key(r)) << 3);
  const int off1 = r * kStreamBK + ((ch ^ swz_key(r) ^ 4) << 3);
  bf16x8 fa[MBV];
#pragma unroll
  for (int m = 0; m < MBV; ++m)
    fa[m] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(&As[2048 * m + ((m & 1) ? off1 : off0)]));
  const bf16x8 w0 = __builtin_bit_cast(bf16x8, bw[0]);
  const bf16x8 w1 = __builtin_bit_cast(bf16x8, bw[1]);
#pragma unroll
  for (int m = 0; m < MBV; ++m) {
    acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, fa[m], acc[m][0], 0, 0, 0);
    acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, fa[m], acc[m][1], 0, 0, 0);
  }
}

// The K loop of one tile.  nxt is the workgroup's next tile if has_next, else
// ignored.  Every tile computes and loads all MBW token blocks (rows past the
// tile's last repeat it), so the loop's load counts are the same for every
// tile and every wait below is a constant.  acc[m][j]: lane l is token 32 m +
// (l mod 32), register r is weight row (block j) + mfma32_row(r, l).
//
// Schedule per K block kb: wait for its LDS stage, barrier, issue the LDS stage
// of block kb + 3, then 4 MFMA steps, each followed by the weight loads of the
// step 16 ahead.  PF = 16 steps = 4 blocks, so in the last 4 blocks of a tile
// every weight refill is the next tile's (steps 0..15) and the LDS stages
// issued in its last 3 blocks are the next tile's blocks 0..2.
//
// next() is called once, before the tile's last 4 blocks (so that the next
// tile's sources are live only while they are needed); it fills nxt and
// returns whether there is a next tile.
template <int BM, typename Next>
__device__ __forceinline__ void stream_tile(const StreamSrc<BM>& cur, StreamSrc<BM>& nxt, Next&& next,
                                            StreamState& ss, const bf16_t* lds,
                                            f32x16 (&acc)[StreamTile<BM>::MBW][2]) {
  constexpr int NS = kStreamNS;
  constexpr int PF = kStreamPF;
  constexpr int MBW = StreamTile<BM>::MBW;
  static_assert(NS == 4 && PF == 16, "the schedule below is written for 4 stages and 16 steps");
  // loads a wave issues per K block: MBW LDS loads and 8 weight loads.  The
  // stage of block kb was issued 3 blocks earlier; after it came 3 x 8 weight
  // loads and the MBW LDS loads of 2 later stages.
  constexpr int kKeep = 8 * (NS - 1) + 2 * MBW;
  const int lane = threadIdx.x & 63;
  const int NKB = cur.nkb;
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    acc[m][0] = f32x16{0.f};
    acc[m][1] = f32x16{0.f};
  }
  bool has_next = false;
  const bf16_t* tail_w[2] = {cur.w[0], cur.w[1]};
  int tail_stride = 0;

  auto kblock = [&](int kb, auto u_tag, auto last_tag) {
    constexpr int u = decltype(u_tag)::value;        // ring slots 4u .. 4u + 3
    constexpr bool last = decltype(last_tag)::value; // one of the tile's last 4 blocks
    // wait for this block's stage; in the last blocks the later stages may be
    // the next tile's, or none after the last tile
    if constexpr (last && u == 3) {
      if (has_next) __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(8 * (NS - 1)));
    } else if constexpr (last && u == 2) {
      if (has_next) __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(8 * (NS - 1) + MBW));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
    }
    __builtin_amdgcn_s_barrier();
    // refill the stage read in the previous block with block kb + 3
    {
      const int dst_st = ss.st == 0 ? NS - 1 : ss.st - 1;
      const uint32_t dst = stream_stage_addr<BM>(lds, dst_st);
      if constexpr (!last || u == 0) {
        stream_issue(cur, kb + NS - 1, dst);
      } else {
        if (has_next) stream_issue(nxt, u - 1, dst);
      }
    }
    const bf16_t* As = lds + ss.st * StreamTile<BM>::kAElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      constexpr int sl0 = u * 4;                     // == 4 kb mod PF
      const int ch = 2 * i + (lane >> 5);
      stream_step<MBW, MBW>(As, ch, ss.bq[sl0 + i], acc);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16_t* src = last ? tail_w[j] + (sl0 + i) * tail_stride : cur.w[j] + (4 * kb + i + PF) * 512;
        ss.bq[sl0 + i][j] = *reinterpret_cast<const u32x4*>(src + lane * 8);
      }
      // keep each refill right after the step that frees its registers: the
      // scheduler would otherwise sink the loads and shorten the prefetch
      __builtin_amdgcn_sched_barrier(0);
    }
    ss.st = ss.st + 1 == NS ? 0 : ss.st + 1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using No = std::false_type;
  using Yes = std::true_type;
  int kb = 0;
  for (; kb < NKB - 4; kb += 4) {                    // NKB is a multiple of 4
    kblock(kb, I0{}, No{});
    kblock(kb + 1, I1{}, No{});
    kblock(kb + 2, I2{}, No{});
    kblock(kb + 3, I3{}, No{});
  }
  // weight source of refills in the last 4 blocks: the next tile's steps
  // 0..15, or (last tile) a repeat of this tile's last step
  has_next = next();
#pragma unroll
  for (int j = 0; j < 2; ++j) tail_w[j] = has_next ? nxt.w[j] : cur.w[j] + (4 * NKB - 1) * 512;
  tail_stride = has_next ? 512 : 0;
  kblock(kb, I0{}, Yes{});
  kblock(kb + 1, I1{}, Yes{});
  kblock(kb + 2, I2{}, Yes{});
  kblock(kb + 3, I3{}, Yes{});
}

}  // namespace moe
