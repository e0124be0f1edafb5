// Main loop of the grouped GEMMs: weights streamed from HBM straight into MFMA
// registers, token rows staged in LDS, one continuous stream across the tiles
// a persistent workgroup computes.
//
// A workgroup of 4 waves computes, for a tile of BM token rows and 4 x 32 NB
// weight rows, C^T = W A^T with v_mfma_f32_32x32x16_bf16 (fp32 accumulation).
// Wave w owns NB 32-row weight blocks and all BM rows, so each A fragment read
// from LDS feeds NB MFMAs: NB = 2 for weight-stream-bound shapes (tall token
// tiles, so an expert's weights stream once), NB = 4 where MFMA throughput is
// the limit (half the LDS reads per MFMA).
//   * Weights are stored packed in MFMA fragment order (moe_pack_weights): the
//     operand of one wave for one 32-row block and one 16-wide K step is 1 KB
//     of contiguous memory, lane l holding 16 bytes.  Each wave streams its
//     blocks with whole-line 16-byte loads into a ring of PF steps (4, 8 or
//     16) of registers -- register space is far larger than LDS, so many bytes are in
//     flight per CU, which is what an HBM-bound stream needs.
//   * FP8 weights (W8): one 1 KB load per block holds the E4M3 codes of two
//     16-wide K steps (8 bytes per lane each, moe_quantize_weights_fp8's
//     layout); they are widened to bf16 in registers (exact) just before their
//     MFMAs, so a ring step covers 2 K steps instead of 1.
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
//     repeat it, so their results repeat its results): the per-block load
//     counts are then the same for every tile, every wait is a compile-time
//     constant, and one set of registers holds the weight ring for all tiles.
// The weight operand is the MFMA's first operand: in an accumulator lane l holds
// token (l mod 32) of its block and register quad q four consecutive weight
// rows; the epilogues pair lanes l and l + 32 so that each stores eight adjacent
// outputs of one token.
#pragma once

#include <type_traits>

#include "lds_dma.h"

namespace moe {

constexpr int kStreamBK = 64;        // K per LDS stage (4 MFMA steps)
constexpr int kStreamNS = 4;         // LDS stages
constexpr int kStreamKAlign = 256;   // every K is a multiple (4 blocks, PF <= 16 steps)

// Ring steps (1 KB weight loads per block) per K block of 64: 4 for bf16
// weights, 2 for FP8 ones.
template <bool W8>
constexpr int kRingPerBlock = W8 ? 2 : 4;

template <int BM, int NB, int PF, bool W8 = false>
struct StreamTile {
  static constexpr int MBW = BM / 32;             // token blocks (every wave covers all)
  static constexpr int kAElems = BM * kStreamBK;  // one LDS stage
  // the ring must fit in the last 4 blocks of a tile (they prefetch the next
  // tile's first PF steps)
  static_assert((NB == 2 || NB == 4) && MBW >= 1 && MBW <= 8 && (PF == 4 || PF == 8 || PF == 16) &&
                    PF <= 4 * kRingPerBlock<W8>,
                "tile shape");
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
template <int MBW>
__device__ __forceinline__ int stream_a_slot(int g, int wave, int lane) {
  return (wave * MBW + g) * 64 + lane;
}

// Sources of one tile.  Everything but a_off is the same in every lane.
template <int BM, int NB>
struct StreamSrc {
  const bf16_t* a_base;                 // token rows: this lane's chunk of group g
  uint32_t a_off[BM / 32];              //   at K = 0 is at a_base + a_off[g] bytes
  const unsigned char* w[NB];           // the wave's packed weight blocks (1 KB per ring step)
  int nkb;                              // K / 64, a multiple of 4
};

// Weight load (1 KB) of block j for ring step `step`.
template <int BM, int NB>
__device__ __forceinline__ const unsigned char* stream_wstep(const StreamSrc<BM, NB>& s, int j, int step) {
  return s.w[j] + step * 1024;
}

// One 16-byte weight load.  NT: a non-temporal load, for weights that no
// other tile of the launch reads again (the line is not kept in L2 / MALL at the
// expense of the token rows and outputs that are).
template <bool NT>
__device__ __forceinline__ u32x4 load_weights(const unsigned char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

// Whether a tile shape's weight loads are non-temporal: the tall and short
// row blocks meant for up to ~200 rows per expert, where an expert's rows
// mostly sit in one block and its weights stream once per launch.
template <int BM>
constexpr bool kStreamWeightsOnce = BM != 96;

// What stays in flight between tiles.
template <int NB, int PF>
struct StreamState {
  u32x4 bq[PF][NB];                     // weight operands of the next PF steps
  int st;                               // LDS stage holding the next K block
};

// The LDS stage of K block kb: all MBW 32-row groups.
template <int BM, int NB>
__device__ __forceinline__ void stream_issue(const StreamSrc<BM, NB>& s, int kb, uint32_t dst) {
  const bf16_t* base = s.a_base + kb * kStreamBK;
#pragma unroll
  for (int g = 0; g < BM / 32; ++g) dma16_off(base, s.a_off[g], dst + g * 1024);
}

template <int BM>
__device__ __forceinline__ uint32_t stream_stage_addr(const bf16_t* lds, int st) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return lds_addr(lds + st * (BM * kStreamBK) + (stream_a_slot<BM / 32>(0, wave, 0) << 3));
}

// Starts the stream with the first tile: its first NS - 1 token-row blocks,
// then its first PF weight steps in step order (the compiler derives the wait
// before each step from the order it sees on entry to the loop).
template <int BM, int NB, int PF>
__device__ __forceinline__ void stream_start(const StreamSrc<BM, NB>& s, StreamState<NB, PF>& ss, const bf16_t* lds) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int st = 0; st < kStreamNS - 1; ++st) stream_issue(s, st, stream_stage_addr<BM>(lds, st));
  ss.st = 0;
#pragma unroll
  for (int p = 0; p < PF; ++p) {
#pragma unroll
    for (int j = 0; j < NB; ++j) ss.bq[p][j] = load_weights<kStreamWeightsOnce<BM>>(stream_wstep(s, j, p) + lane * 16);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Drains the stream after the last tile (its tail loads repeat the last step).
__device__ __forceinline__ void stream_finish() {
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

// A fragments of the MBW token blocks for 16-wide step `ch / 2` of an LDS
// stage.  pipe_swz(32 m + r, ch) = 2048 m + r * 64 + ((ch ^ swz_key(r) ^
// 4 (m & 1)) << 3) for r < 32: two lane offsets serve every block (the rest is
// an immediate).
template <int MBW>
__device__ __forceinline__ void stream_read_a(const bf16_t* As, int ch, bf16x8 (&fa)[MBW]) {
  const int r = threadIdx.x & 31;
  const int off0 = r * kStreamBK + ((ch ^ swz_key(r)) << 3);
  const int off1 = r * kStreamBK + ((ch ^ swz_key(r) ^ 4) << 3);
#pragma unroll
  for (int m = 0; m < MBW; ++m)
    fa[m] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(&As[2048 * m + ((m & 1) ? off1 : off0)]));
}

// One MFMA step: NB MFMAs per token block.
template <int MBW, int NB>
__device__ __forceinline__ void stream_mfma(const bf16x8 (&fa)[MBW], const bf16x8 (&bw)[NB],
                                            f32x16 (&acc)[MBW][NB]) {
#pragma unroll
  for (int m = 0; m < MBW; ++m)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[j], fa[m], acc[m][j], 0, 0, 0);
}

// Eight E4M3 codes (two dwords, byte i = K element i) -> the bf16 MFMA operand
// (exact: every E4M3 value is a bf16 value; scale 1).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The K loop of one tile.  Every tile computes and loads all MBW token blocks
// (rows past the tile's last repeat it), so the loop's load counts are the
// same for every tile and every wait below is a constant.  acc[m][j]: lane l
// is token 32 m + (l mod 32), register r is weight row (block j) +
// mfma32_row(r, l).
//
// Schedule per K block kb: wait for its LDS stage, barrier, issue the LDS stage
// of block kb + 3, then 4 MFMA steps, each followed by the weight loads of the
// step PF ahead.  The tile's last 4 blocks are unrolled: their LDS issues are
// this tile's last block, then the next tile's blocks 0..2, and their weight
// refills past this tile's last step are the next tile's first steps.
//
// next() is called once, before the tile's last 4 blocks (so that the next
// tile's sources are live only while they are needed); it fills nxt and
// returns whether there is a next tile.
//
// stored: the caller issued exactly ST vector-memory stores per wave after the
// previous tile's loop (its epilogue).  Those stores sit between the LDS
// stages of blocks 0..2 (issued in the previous tile's last blocks) and their
// waits, so these waits count them too; vector-memory operations of a wave
// retire in issue order (loads and stores alike), so a wait that counts them
// still guarantees its stage has landed and no longer drains the loads issued
// after it.  A count past the counter's range falls back to the plain wait.
template <int BM, int NB, int PF, bool W8, int ST, typename Next, typename Hook>
__device__ __forceinline__ void stream_tile(const StreamSrc<BM, NB>& cur, StreamSrc<BM, NB>& nxt, Next&& next,
                                            Hook&& tail_hook, StreamState<NB, PF>& ss, const bf16_t* lds,
                                            f32x16 (&acc)[BM / 32][NB], bool stored) {
  constexpr int NS = kStreamNS;
  constexpr int MBW = BM / 32;
  constexpr int RSB = kRingPerBlock<W8>;             // ring steps per K block
  constexpr int U = PF / RSB;                        // blocks per unrolled body
  static_assert(NS == 4 && StreamTile<BM, NB, PF, W8>::MBW == MBW && U >= 1 && PF % RSB == 0,
                "the schedule below is written for 4 stages");
  // loads a wave issues per K block: MBW LDS loads and RSB NB weight loads.
  // The stage of block kb was issued 3 blocks earlier; after it came 3 x RSB NB
  // weight loads and the MBW LDS loads of 2 later stages.
  constexpr int kW = RSB * NB * (NS - 1);
  constexpr int kKeep = kW + 2 * MBW;
  static_assert(kKeep < 64, "vmcnt range");
  constexpr int kStoreComp = kKeep + ST <= 63 ? ST : 0;   // added to the waits of blocks 0..2
  const int lane = threadIdx.x & 63;
  const int NKB = cur.nkb;
#pragma unroll
  for (int m = 0; m < MBW; ++m)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[m][j] = f32x16{0.f};
  bool has_next = false;
  const unsigned char* tail_w[NB];
  int tail_stride = 0;
#pragma unroll
  for (int j = 0; j < NB; ++j) tail_w[j] = cur.w[j];

  // u: position of the block in its unrolled group (ring slots RSB u .. RSB u +
  // RSB - 1 mod PF)
  auto kblock = [&](int kb, auto u_tag, auto last_tag) {
    constexpr int u = decltype(u_tag)::value;
    constexpr bool last = decltype(last_tag)::value; // u-th of the tile's last 4 blocks
    // wait for this block's stage; in the last blocks the later stages may be
    // the next tile's, or none after the last tile
    const bool comp = kStoreComp > 0 && stored && kb < NS - 1;
    if constexpr (last && u == 3) {
      if (has_next) {
        if (comp) __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep + kStoreComp));
        else __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
      } else {
        if (comp) __builtin_amdgcn_s_waitcnt(vmcnt_only(kW + kStoreComp));
        else __builtin_amdgcn_s_waitcnt(vmcnt_only(kW));
      }
    } else if constexpr (last && u == 2) {
      if (has_next) {
        if (comp) __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep + kStoreComp));
        else __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
      } else {
        if (comp) __builtin_amdgcn_s_waitcnt(vmcnt_only(kW + MBW + kStoreComp));
        else __builtin_amdgcn_s_waitcnt(vmcnt_only(kW + MBW));
      }
    } else {
      if (comp) __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep + kStoreComp));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(kKeep));
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
    if constexpr (last) tail_hook(u_tag);
    const bf16_t* As = lds + ss.st * (BM * kStreamBK);
    bf16x8 w8op[NB][2];                                // W8: the two K steps of a ring step
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rs = W8 ? i >> 1 : i;                  // ring step inside the block
      const int slot = (RSB * u + rs) % PF;            // == (RSB kb + rs) mod PF
      bf16x8 fa[MBW];
      stream_read_a<MBW>(As, 2 * i + (lane >> 5), fa);
      bf16x8 bw[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (W8) {
          if ((i & 1) == 0) {
            w8op[j][0] = fp8x8_to_bf16x8(ss.bq[slot][j][0], ss.bq[slot][j][1]);
            w8op[j][1] = fp8x8_to_bf16x8(ss.bq[slot][j][2], ss.bq[slot][j][3]);
          }
          bw[j] = w8op[j][i & 1];
        } else {
          bw[j] = __builtin_bit_cast(bf16x8, ss.bq[slot][j]);
        }
      }
      stream_mfma<MBW, NB>(fa, bw, acc);
      // the ring step PF ahead, once this one's registers are free: this
      // tile's, or in the last blocks past its end the next tile's (every
      // tile has at least 4 RSB ring steps)
      if (!W8 || (i & 1) == 1) {
        const bool from_next = last && (RSB * u + rs + PF >= 4 * RSB);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const unsigned char* src = from_next ? tail_w[j] + (RSB * u + rs + PF - 4 * RSB) * tail_stride
                                               : stream_wstep(cur, j, RSB * kb + rs + PF);
          ss.bq[slot][j] = load_weights<kStreamWeightsOnce<BM>>(src + lane * 16);
        }
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
  for (; kb < NKB - 4; kb += U) {                    // NKB is a multiple of 4
    kblock(kb, I0{}, No{});
    if constexpr (U >= 2) kblock(kb + 1, I1{}, No{});
    if constexpr (U == 4) {
      kblock(kb + 2, I2{}, No{});
      kblock(kb + 3, I3{}, No{});
    }
  }
  // weight source of refills past this tile's last step: the next tile's first
  // steps, or (last tile) a repeat of one step of this tile
  has_next = next();
#pragma unroll
  for (int j = 0; j < NB; ++j) tail_w[j] = has_next ? nxt.w[j] : cur.w[j];
  tail_stride = has_next ? 1024 : 0;
  kblock(kb, I0{}, Yes{});
  kblock(kb + 1, I1{}, Yes{});
  kblock(kb + 2, I2{}, Yes{});
  kblock(kb + 3, I3{}, Yes{});
}

}  // namespace moe
