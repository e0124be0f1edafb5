// Grouped GEMMs for batches with many rows per expert: 256 x 256 tiles with
// both operands staged in LDS, bf16 MFMA with fp32 accumulation.
//
// What they compute is what grouped_gemm.hip computes ("Laguna-M.1-base",
// Feed-forward: SwiGLU without biases; the grouped GEMM over expert-ordered
// tokens of "Laguna M.1/XS.2 Technical Report", Key claims, report section
// 3.1.2):  gate_up  h[p] = silu(Wg_e a_p) * (Wu_e a_p),  down  y[p] = Wd_e h[p],
// the shared expert as one more group over all T rows; the plain mode (down)
// also serves the training pass's products.
//
// Why a second kernel: once an expert has a few hundred rows the MFMA pipes,
// not the HBM weight stream, set the pace, and the limit becomes the bytes a
// CU pulls through its load path per MFMA.  A tile of 256 token rows x 256
// weight rows with both operands in LDS pulls 0.25 KB per 32x32x16 MFMA (32
// bytes per clock per CU at the full MFMA rate), which the load path sustains
// from L2 (about 45-50 bytes per clock per CU measured on this part), provided
// that the tiles sharing operands run together behind one L2.
//
// Design:
//   * persistent grid, one workgroup of 4 waves per CU; the tile table is built
//     on the device from `offsets` (no host synchronisation); the shared group's
//     tiles come first, then the routed experts'; inside a group the output
//     column blocks of one row block are adjacent, and tiles go out in rounds of
//     one per workgroup, each round cut into 8 runs of consecutive tiles, one
//     run per XCD, so the tiles of one expert run at the same time behind one
//     L2 and walk K in step;
//   * waves in a 2 x 2 grid: wave (r, c) owns 4 token blocks x 4 weight blocks
//     of 32 (256 fp32 accumulators per lane); token block b of the tile goes to
//     wave row b mod 2, so a ragged last row block of an expert splits its
//     blocks evenly over both wave rows, and a wave skips the MFMAs of blocks
//     that hold no row;
//   * K advances in stages of 32, filled by direct global->LDS loads
//     (global_load_lds_dwordx4): the weights of a stage (packed 1 KB MFMA
//     operand blocks, 16 KB) go through a ring of 4 buffers; the token rows go
//     in pairs of stages, 64 K values = one whole 128-byte line per row (a
//     wave load: 8 rows), through 2 buffers of 32 KB, XOR-swizzled for
//     conflict-free ds_read_b128.  Rows gathered through `sorted_token` are
//     scattered over the activations, and a 1 KB wave load of whole lines
//     touches 8 lines where one of 64-byte rows (one stage) touches 16
//     (measured: gate/up 2%, down 4% faster on the long prefill);
//   * one barrier per stage, between its two MFMA steps: by then every wave has
//     read the stage before it (whose weight buffer then takes the stage three
//     ahead; in an odd stage, the pair buffer of the stage and the one before
//     it takes the pair three and four ahead) and each wave has waited for its
//     own loads of the next stage; MFMA operands are read from LDS one step
//     ahead into a second register set;
//   * the rings do not drain between tiles: the last stages of a tile load the
//     next tile's first three stages, and the tile's outputs are stored after
//     them (a constant number of 16-byte stores per wave: rows past a tile's
//     last rewrite its last row, skipped blocks rewrite the wave's first block,
//     with the same bits), so the next tile's first waits can count them;
//   * gate_up pairs each wave's two gate blocks with the up blocks of the same
//     columns, so SwiGLU is applied in registers before one rounding to bf16;
//   * outputs leave through LDS (the wave's 4 KB of the tile's last weight
//     buffer), so that every store writes whole 128-byte row segments; down's
//     stores are non-temporal (the combine reads them once, later).
#include "grouped_gemm.h"
#include <utility>

#include "mma_stream.h"

namespace moe {
namespace {

constexpr int kLThreads = 256;
constexpr int kLBM = 256;                 // token rows per tile
constexpr int kLBN = 256;                 // weight rows per tile
constexpr int kLBK = 32;                  // K per LDS stage (two 16-wide MFMA steps)
constexpr int kLNS = 4;                   // weight buffers of the ring (one K stage each)
constexpr int kLPairA = kLBM * 2 * kLBK * 2;   // 32 KB: token rows of two K stages (128 bytes a row)
constexpr int kLStageB = kLBN * kLBK * 2;      // 16 KB of weight blocks per stage
constexpr int kLBOff = 2 * kLPairA;            // the weight ring follows the two token-row pair buffers

// Chunk swizzle of a 128-byte token row (a pair of stages) in LDS: 16-byte
// chunk c of tile row r sits at slot c ^ lswz8(r).  A ds_read_b128 of 32 rows,
// one chunk each, then hits distinct slots in every group of 16 consecutive
// rows (8 pairs of rows, each pair one 256-byte bank window).
__device__ __forceinline__ int lswz8(int r) { return (r >> 1) & 7; }

// s_waitcnt immediate that waits for lgkmcnt <= n only (gfx9 encoding).
constexpr int lgkmcnt_only(int n) { return 15 | (7 << 4) | ((n & 15) << 8) | (3 << 14); }

// The order in which a step's MFMAs first use its operands (token block 0,
// weight blocks 0-3, token blocks 1-3): read r of a step fetches operand
// op_order(r).
constexpr int op_order(int r) { return r == 0 ? 0 : (r <= 4 ? 3 + r : r - 4); }

// Sources of one tile (everything uniform except a_off).
struct LTile {
  const unsigned char* a;      // token rows: the chunk of load i of pair q (K stages 2q, 2q + 1) is at a + 128 q + a_off[i]
  uint32_t a_off[8];
  const unsigned char* w[2];   // the wave's two weight blocks: K stage kb, step s at w[j] + 2048 kb + 1024 s
  int nkb;                     // K / 32
  int nv;                      // token blocks of this wave that hold rows (1..4)
  int tb0;                     // tile block of the wave's first block (the wave row, or 0)
  bf16_t* out;                 // output element (tile row r, column c of the wave) at out + r * ld + c
  int ld;
  int valid;                   // rows of the tile
  int gathered;                // token rows gathered through the expert order
  const int32_t* ids;          // gathered: the tile's token ids (rows past valid - 1 repeat its last)
  int K;                       // reduction length (elements)
};

// A pointer that is the same in every lane, made visibly so (SGPRs).
template <typename T>
__device__ __forceinline__ const T* uni(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One direct global->LDS load: 16 bytes per lane from base + voff (lane l's
// bytes land at LDS byte lds + off + 16 l).  base and lds are uniform (SGPRs),
// off a constant.  The scalar add that forms m0 writes SCC, so SCC is listed
// as clobbered (a carry the compiler keeps live across the block, between the
// halves of a 64-bit address add, would otherwise be overwritten).
template <int OFF>
__device__ __forceinline__ void dma_lds(const unsigned char* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds), "i"(OFF)
               : "memory", "m0", "scc");
}

template <int MODE>
__global__ __launch_bounds__(kLThreads, 1) void lds_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLBOff + kLNS * kLStageB];
  __shared__ int tile_end[kGemmMaxE + 1];
  __shared__ int row_base[kGemmMaxE + 1];
  __shared__ __attribute__((aligned(256))) int32_t ids_lds[4][64];   // next tile's token ids, per wave
  static_assert(kLBOff + kLNS * kLStageB + 2 * (kGemmMaxE + 1) * 4 + 4 * 64 * 4 <= 160 * 1024, "LDS");
  constexpr int kOutCols = MODE == kGateUp ? kLBN / 2 : kLBN;    // output columns per tile
  constexpr int kJ = MODE == kGateUp ? 2 : 4;                    // output blocks of 32 per wave
  constexpr int kStores = 4 * kJ * 2;                            // 16-byte stores per wave and tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int E = g.E;
  const int nt_r = g.N / kOutCols;
  const int nt_s = g.has_shared ? g.Ns / kOutCols : 0;
  const int n_sh = g.has_shared ? (g.T + kLBM - 1) / kLBM * nt_s : 0;
  const int G = gridDim.x;

  // ---- tile table of the routed groups: tiles per expert, inclusive scan
  {
    int cnt = 0;
    if (tid < E) {
      // clamped so that no offsets table can move a tile outside [0, S)
      const int lo = min(max(g.offsets[tid], 0), g.S);
      const int hi = min(max(g.offsets[tid + 1], lo), g.S);
      row_base[tid] = lo;
      cnt = (hi - lo + kLBM - 1) / kLBM * nt_r;
    }
    const int ln = tid & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(cnt, d);
      if (ln >= d) cnt += v;
    }
    if (ln == 63) tile_end[tid] = cnt;
    __syncthreads();
    for (int w = 0; w < (tid >> 6); ++w) cnt += tile_end[64 * w + 63];
    __syncthreads();
    tile_end[tid] = cnt;
    if (tid == 0) row_base[E] = E > 0 ? min(max(g.offsets[E], row_base[E - 1]), g.S) : 0;
    __syncthreads();
  }
  const int total = n_sh + (E > 0 ? __builtin_amdgcn_readfirstlane(tile_end[E - 1]) : 0);

  // ---- rounds of G tiles, each cut into 8 runs of consecutive tiles, one per
  // XCD (workgroup b runs on XCD b mod 8); a short last round is split evenly
  // over the XCDs
  const int xcd = blockIdx.x % kGemmXcds, in_xcd = blockIdx.x / kGemmXcds;
  auto tile_at = [&](int r) -> int {
    const int base = r * G;
    if (base >= total) return -1;
    const int n = min(G, total - base);
    if (n == G) return base + xcd * (G / kGemmXcds) + in_xcd;
    const int q = n / kGemmXcds, rem = n % kGemmXcds;
    if (in_xcd >= q + (xcd < rem ? 1 : 0)) return -1;
    return base + xcd * q + min(xcd, rem) + in_xcd;
  };

  // ---- where a tile sits: group (E: the shared expert), its first row and
  // row count, the tile's origin
  struct Where {
    int grp, rb, M, m0, n0;
  };
  auto locate = [&](int ti) __attribute__((always_inline)) {
    const bool shared = ti < n_sh;
    int grp = E, local = ti;
    if (!shared) {
      const int r = ti - n_sh;
      int lo = 0, hi = E - 1;         // first group with tile_end > r
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tile_end[mid] > r) hi = mid; else lo = mid + 1;
      }
      grp = lo;
      local = r - (grp == 0 ? 0 : tile_end[grp - 1]);
    }
    const int nt = max(1, shared ? nt_s : nt_r);
    local = max(local, 0);
    Where w;
    w.grp = grp;
    w.rb = shared ? 0 : row_base[grp];
    w.M = shared ? g.T : row_base[grp + 1] - w.rb;
    w.m0 = (local / nt) * kLBM;
    w.n0 = (local % nt) * kOutCols;
    return w;
  };
  // The down projection's tiles are short (K = F), so walking the tile table
  // for each one (a chain of dependent LDS and scalar loads at the tile top)
  // weighs more there: lane l of each wave locates the tile of round r0 + l,
  // 64 rounds at a time, and a tile's decode reads its entry with v_readlane
  // (d_grp -1: no tile; measured: down 1-2% faster on the long prefill and at
  // the M.1 widths, results bit for bit the same).  Gate/up (K = D, 4x longer
  // tiles) walks the table per tile: the batch's registers made it 1% slower.
  constexpr bool kBatch = MODE == kDown;
  int d_grp = 0, d_rb = 0, d_M = 0, d_m0 = 0, d_n0 = 0;
  auto fill_batch = [&](int r0) {
    const int ti = tile_at(r0 + lane);
    const Where w = locate(max(ti, 0));
    d_grp = ti < 0 ? -1 : w.grp;
    d_rb = w.rb;
    d_M = w.M;
    d_m0 = w.m0;
    d_n0 = w.n0;
  };

  // ---- sources and output of the tile of round r (slot ti)
  auto decode = [&](int r, int ti, LTile& t) __attribute__((always_inline)) {
    int ln = tid & 63;
    asm volatile("" : "+v"(ln));      // per-lane arithmetic stays inside decode
    int grp, rb, M, m0, n0;
    bool shared;
    if constexpr (kBatch) {
      const int sl = r & 63;
      grp = __builtin_amdgcn_readlane(d_grp, sl);
      shared = grp == E;
      rb = __builtin_amdgcn_readlane(d_rb, sl);
      M = __builtin_amdgcn_readlane(d_M, sl);
      m0 = __builtin_amdgcn_readlane(d_m0, sl);
      n0 = __builtin_amdgcn_readlane(d_n0, sl);
    } else {
      const bool sh = ti < n_sh;
      shared = sh;
      int local = ti, first = 0;
      grp = E;
      if (!sh) {
        const int r = ti - n_sh;
        int lo = 0, hi = E - 1;       // first group with tile_end > r
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (tile_end[mid] > r) hi = mid; else lo = mid + 1;
        }
        grp = __builtin_amdgcn_readfirstlane(lo);
        first = grp == 0 ? 0 : __builtin_amdgcn_readfirstlane(tile_end[grp - 1]);
        local = r - first;
      }
      rb = sh ? 0 : __builtin_amdgcn_readfirstlane(row_base[grp]);
      M = sh ? g.T : __builtin_amdgcn_readfirstlane(row_base[grp + 1]) - rb;
      const int nt = sh ? nt_s : nt_r;
      m0 = (local / nt) * kLBM;
      n0 = (local % nt) * kOutCols;
    }
    const int K = shared ? g.Ks : g.K;
    const int Nout = shared ? g.Ns : g.N;
    const int valid = min(kLBM, M - m0);
    const int mb = (valid + 31) >> 5;                    // token blocks that hold rows
    const int nv_raw = wr == 0 ? (mb + 1) >> 1 : mb >> 1;
    t.nv = nv_raw > 0 ? nv_raw : 1;
    t.tb0 = nv_raw > 0 ? wr : 0;
    t.nkb = K / kLBK;
    t.valid = valid;

    // token rows: load i of this wave fills tile rows 64 wave + 8 i + 0..7,
    // lane l row 64 wave + 8 i + l / 8, LDS slot l % 8 = logical chunk
    // (l % 8) ^ lswz8(row); rows past the tile's last repeat it
    const bool gathered = !shared && g.gather != nullptr;
    t.gathered = gathered;
    t.K = K;
    t.ids = gathered ? uni(g.gather + rb + m0) : nullptr;
    if (gathered) {
      // token ids arrive later through LDS (ids_issue / ids_offsets)
      t.a = uni(reinterpret_cast<const unsigned char*>(g.a_routed));
    } else {
      t.a = uni(reinterpret_cast<const unsigned char*>(shared ? g.a_shared + static_cast<size_t>(m0) * K
                                                              : g.a_routed + static_cast<size_t>(rb + m0) * K));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + (ln >> 3);
        const int c = (ln & 7) ^ lswz8(row);
        const int r = min(row, valid - 1);
        t.a_off[i] = (static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + 8u * c) * 2u;
      }
    }
    // weight blocks this wave loads: tile weight blocks 2 wave and 2 wave + 1
    // (gate_up: blocks 0-3 are gate rows n0.., blocks 4-7 the up rows of the
    // same columns)
    const int Nw = MODE == kGateUp ? 2 * Nout : Nout;
    const unsigned char* wmat = shared ? g.w_shared : g.w_routed + static_cast<size_t>(grp) * Nw * K * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = 2 * wave + j;
      const int wrow = MODE == kGateUp ? (blk < 4 ? n0 + 32 * blk : Nout + n0 + 32 * (blk - 4)) : n0 + 32 * blk;
      t.w[j] = uni(wmat + static_cast<size_t>(wrow >> 5) * K * 64);
    }
    // output: the wave's columns
    const int col0 = n0 + (MODE == kGateUp ? 64 : 128) * wc;
    t.out = const_cast<bf16_t*>(uni((shared ? g.out_shared + static_cast<size_t>(m0) * Nout
                                            : g.out_routed + static_cast<size_t>(rb + m0) * Nout) + col0));
    t.ld = Nout;
  };

  // direct loads: the token rows of two K stages (a pair: 64 K values, one
  // whole 128-byte line per row) into one of two pair buffers, load i of 8
  // filling rows 64 wave + 8 i + lane / 8; and the weight blocks of one stage
  // into one of four stage buffers (load i of 4: block i / 2, step i % 2).
  // lbwA / lbwB: the LDS byte address of this wave's first 1 KB slot
  const uint32_t lds0 = lds_addr(smem);
  auto lbwA = [&](int pbuf) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
        lds0 + static_cast<uint32_t>(pbuf) * kLPairA + 8192u * static_cast<uint32_t>(wave)));
  };
  auto lbwB = [&](int buf) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
        lds0 + kLBOff + static_cast<uint32_t>(buf) * kLStageB + 4096u * static_cast<uint32_t>(wave)));
  };
  const uint32_t vb[2] = {static_cast<uint32_t>(lane) * 16u, static_cast<uint32_t>(lane) * 16u + 1024u};
  auto issue_a = [&](const unsigned char* src, const uint32_t (&aoff)[8], uint32_t lb, int i) __attribute__((always_inline)) {
    switch (i) {
      case 0: dma_lds<0>(src, aoff[0], lb); break;
      case 1: dma_lds<1024>(src, aoff[1], lb); break;
      case 2: dma_lds<2048>(src, aoff[2], lb); break;
      case 3: dma_lds<3072>(src, aoff[3], lb); break;
      case 4: dma_lds<4096>(src, aoff[4], lb); break;
      case 5: dma_lds<5120>(src, aoff[5], lb); break;
      case 6: dma_lds<6144>(src, aoff[6], lb); break;
      default: dma_lds<7168>(src, aoff[7], lb); break;
    }
  };
  auto issue_b = [&](const unsigned char* w0, const unsigned char* w1, uint32_t lb, int i) __attribute__((always_inline)) {
    switch (i) {
      case 0: dma_lds<0>(w0, vb[0], lb); break;
      case 1: dma_lds<1024>(w0, vb[1], lb); break;
      case 2: dma_lds<2048>(w1, vb[0], lb); break;
      default: dma_lds<3072>(w1, vb[1], lb); break;
    }
  };
  auto issue_a_all = [&](const LTile& t, int q, int pbuf) {
    const unsigned char* src = uni(t.a + 128 * q);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_a(src, t.a_off, lbwA(pbuf), i);
  };
  auto issue_b_all = [&](const LTile& t, int kb, int buf) {
    const unsigned char* w0 = uni(t.w[0] + 2048 * kb);
    const unsigned char* w1 = uni(t.w[1] + 2048 * kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_b(w0, w1, lbwB(buf), i);
  };

  // Token ids of a gathered tile: one direct load of 4 bytes per lane puts the
  // ids of the wave's 64 rows (64 wave + l, clamped to the tile's last row)
  // into ids_lds[wave]; a tile that gathers nothing (or no tile) loads 256
  // harmless bytes of `dummy` instead, so every tile issues exactly one.
  const uint32_t ids_l = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds_addr(&ids_lds[wave][0])));
  auto ids_issue = [&](const LTile& t, bool real, const unsigned char* dummy) __attribute__((always_inline)) {
    const bool gath = real && t.gathered;
    const unsigned char* base = uni(gath ? reinterpret_cast<const unsigned char*>(t.ids) : dummy);
    const uint32_t voff = gath ? static_cast<uint32_t>(min(64 * wave + lane, t.valid - 1)) * 4u
                               : static_cast<uint32_t>(lane) * 4u;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(ids_l)
                 : "memory", "m0");
  };
  // the row offsets of a gathered tile from its ids in LDS (once its load
  // has landed): load i, lane l reads row 64 wave + 8 i + l / 8
  auto ids_offsets = [&](LTile& t) __attribute__((always_inline)) {
    if (!t.gathered) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 64 * wave + 8 * i + (lane >> 3);
      const int tok = min(max(ids_lds[wave][8 * i + (lane >> 3)], 0), g.T - 1);
      const int c = (lane & 7) ^ lswz8(row);
      t.a_off[i] = (static_cast<uint32_t>(tok) * static_cast<uint32_t>(t.K) + 8u * c) * 2u;
    }
  };

  // LDS byte offsets of this lane's operand chunks: token row (lane mod 32) of
  // a block, chunk 4 par + 2 step + lane / 32 of its pair's 8 (par: the
  // stage's place in its pair); weight block at 1 KB per (block, step)
  const int ar = lane & 31;
  uint32_t a_lane[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int st = 0; st < 2; ++st)
      a_lane[par][st] = static_cast<uint32_t>(128 * ar + 16 * ((4 * par + 2 * st + (lane >> 5)) ^ lswz8(ar)));
  // the wave's weight blocks in the tile: gate_up gate 2c, 2c + 1 and up
  // 4 + 2c, 5 + 2c; down 4c .. 4c + 3
  auto wblk = [&](int j) { return MODE == kGateUp ? (j < 2 ? 2 * wc + j : 2 + 2 * wc + j) : 4 * wc + j; };

  typedef bf16x8 Frag[8];           // 4 token-block operands, then 4 weight-block operands
  // operand Q of a step: Q < 4 token block Q, else weight block Q - 4
  // (pbuf, par: the stage's pair buffer and its place in the pair; buf: its
  // weight buffer)
  auto read_op = [&](int tb0, int pbuf, int par, int buf, int step, int q, Frag& f) __attribute__((always_inline)) {
    if (q < 4) {
      // (blocks past the wave's live ones are read too: in bounds, unused)
      const int tb = q == 0 ? tb0 : 2 * q + wr;
      f[q] = *reinterpret_cast<const bf16x8*>(smem + pbuf * kLPairA + 4096 * tb + a_lane[par][step]);
    } else {
      f[q] = *reinterpret_cast<const bf16x8*>(smem + kLBOff + buf * kLStageB + (2 * wblk(q - 4) + step) * 1024 +
                                              16 * lane);
    }
  };

  if constexpr (kBatch) fill_batch(0);
  const int pos = tile_at(0);
  if (pos < 0) return;
  LTile cur, nxt;
  decode(0, pos, cur);
  ids_issue(cur, true, cur.a);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  ids_offsets(cur);
  int ring = 0;                      // weight buffer of the current tile's stage 0
  int aring = 0;                     // token-row buffer of its pair 0 (stages 0 and 1)
  // stages 0-2, in the order the previous tile's last stages issue them
  // (weights 0, pair 0, weights 1 and 2, pair 1: the weights of stage x + 3
  // are issued in stage x's first step, the pair of stages x + 3 and x + 4 in
  // an odd stage x's second)
  issue_b_all(cur, 0, 0);
  issue_a_all(cur, 0, 0);
  issue_b_all(cur, 1, 1);
  issue_b_all(cur, 2, 2);
  issue_a_all(cur, 1, 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(16));
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
#pragma unroll
  for (int r = 0; r < 8; ++r) read_op(cur.tb0, 0, 0, 0, 0, op_order(r), f0);

  bool stored = false;               // the previous tile's stores came between the token-row
                                     // and the weight halves of this tile's stage 3
  int round = 0;
  for (int ti = pos; ti >= 0;) {
    f32x16 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] = f32x16{0.f};
    ring = __builtin_amdgcn_readfirstlane(ring);
    aring = __builtin_amdgcn_readfirstlane(aring);
    const int nkb = __builtin_amdgcn_readfirstlane(cur.nkb);
    const int nv = __builtin_amdgcn_readfirstlane(cur.nv);
    // the next tile, decoded here where the accumulators hold nothing; its
    // token ids land in LDS behind this tile's first loads (the waits of
    // stages 0 and 1 count the one load, and stage 2's wait covers it)
    if constexpr (kBatch) {
      if (((round + 1) & 63) == 0) fill_batch(round + 1);
    }
    const int tn = tile_at(round + 1);
    const bool has_next = tn >= 0;
    if (has_next) decode(round + 1, tn, nxt);
    else nxt = cur;
    ids_issue(nxt, has_next, cur.a);

    // one 16-wide K step over the wave's NV live token blocks; op(k) is the
    // memory operation issued after the k-th MFMA (k = 0..15; the ones past
    // a short step's MFMAs follow them), so the loads' and the LDS reads'
    // issue overlaps the MFMA pipe
    auto step = [&](const Frag& f, auto nv_tag, auto&& op) __attribute__((always_inline)) {
      constexpr int NV = decltype(nv_tag)::value;
#pragma unroll
      for (int m = 0; m < NV; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[4 + j], f[m], acc[m][j], 0, 0, 0);
          op(4 * m + j);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int k = 4 * NV; k < 16; ++k) op(k);
    };

    // K stage x: step 0 from f0 while reading step 1's operands into f1 and
    // issuing the weights of stage x + 3; barrier; step 1 from f1 while
    // reading stage x + 1's first operands into f0 and, in an odd stage,
    // issuing the token rows of stages x + 3 and x + 4 (one pair).  Stages
    // past this tile's last are the next tile's; after the last tile they
    // repeat this tile's first ones (in bounds, never used), so that every
    // stage issues the same loads and waits.  PAR = x mod 2 (K has a multiple
    // of 64 values, so a tile's stage count is even).
    auto stage = [&](int x, auto par_tag, auto nv_tag) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_tag)::value;
      const int b0 = (ring + x) & (kLNS - 1);
      const int b1 = (b0 + 1) & (kLNS - 1);
      const int b3 = (b0 + kLNS - 1) & (kLNS - 1);
      const int p0 = (aring + (x >> 1)) & 1;           // stage x's token-row buffer
      const int p1 = PAR ? p0 ^ 1 : p0;                // stage x + 1's
      const uint32_t l3 = lbwB(b3);
      const bool wnx = x + 3 >= nkb;
      const int wk = wnx ? x + 3 - nkb : x + 3;
      const unsigned char* w0 = uni((wnx ? nxt.w[0] : cur.w[0]) + 2048 * wk);
      const unsigned char* w1 = uni((wnx ? nxt.w[1] : cur.w[1]) + 2048 * wk);
      // the next tile's row offsets, before its first token-row load (step 1
      // of stage nkb - 3); its ids landed by stage 2's wait (nkb >= 8)
      if (x == nkb - kLNS && has_next) ids_offsets(nxt);
      step(f0, nv_tag, [&](int k) __attribute__((always_inline)) {
        if ((k & 1) == 0) read_op(cur.tb0, p0, PAR, b0, 1, op_order(k >> 1), f1);
        else if ((k & 3) == 1) issue_b(w0, w1, l3, k >> 2);
      });
      // stage x + 1 has landed once no more than the loads issued after its
      // last one are outstanding: even x, the weights of stages x + 2 and
      // x + 3 and the pair of x + 3, x + 4 (16); odd x, the weights of x + 2
      // and x + 3 (8); stages 0 and 1 also count the next tile's id load and
      // the previous tile's stores
      if constexpr (PAR == 0) {
        if (x == 0) {
          if (stored) __builtin_amdgcn_s_waitcnt(vmcnt_only(17 + kStores));
          else __builtin_amdgcn_s_waitcnt(vmcnt_only(17));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_only(16));
        }
      } else {
        if (x == 1) {
          if (stored) __builtin_amdgcn_s_waitcnt(vmcnt_only(9 + kStores));
          else __builtin_amdgcn_s_waitcnt(vmcnt_only(9));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_only(8));
        }
      }
      // every wave's reads of stage x were issued by its first step: done
      // before the barrier hands its buffers on
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      __builtin_amdgcn_s_barrier();
      const int tb0 = x + 1 >= nkb ? nxt.tb0 : cur.tb0;
      if constexpr (PAR == 1) {
        // the pair of stages x + 3, x + 4 goes where stages x - 1, x were
        const int q = (x + 3) >> 1;
        const bool anx = q >= (nkb >> 1);
        const int aq = anx ? q - (nkb >> 1) : q;
        const unsigned char* asrc = uni((anx ? nxt.a : cur.a) + 128 * aq);
        uint32_t aoff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) aoff[i] = anx ? nxt.a_off[i] : cur.a_off[i];
        const uint32_t la = lbwA(p0);
        step(f1, nv_tag, [&](int k) __attribute__((always_inline)) {
          if ((k & 1) == 0) read_op(tb0, p1, 0, b1, 0, op_order(k >> 1), f0);
          else issue_a(asrc, aoff, la, k >> 1);
        });
      } else {
        step(f1, nv_tag, [&](int k) __attribute__((always_inline)) {
          if ((k & 1) == 0) read_op(tb0, p1, 1, b1, 0, op_order(k >> 1), f0);
        });
      }
    };

    // two stages x, x + 1 (x even) whose loads all come from this tile and
    // whose waits count no stores: the same work from pointers advanced once
    // per stage
    auto fast = [&](int x, const unsigned char*& pa, const unsigned char*& pw0, const unsigned char*& pw1,
                    auto nv_tag) __attribute__((always_inline)) {
      const int b0 = (ring + x) & (kLNS - 1);
      const int b1 = (b0 + 1) & (kLNS - 1);
      const int b2 = (b0 + 2) & (kLNS - 1);
      const int b3 = (b0 + kLNS - 1) & (kLNS - 1);
      const int p0 = (aring + (x >> 1)) & 1;
      const uint32_t l3 = lbwB(b3);
      step(f0, nv_tag, [&](int k) __attribute__((always_inline)) {
        if ((k & 1) == 0) read_op(cur.tb0, p0, 0, b0, 1, op_order(k >> 1), f1);
        else if ((k & 3) == 1) issue_b(pw0, pw1, l3, k >> 2);
      });
      __builtin_amdgcn_s_waitcnt(vmcnt_only(16));
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      __builtin_amdgcn_s_barrier();
      step(f1, nv_tag, [&](int k) __attribute__((always_inline)) {
        if ((k & 1) == 0) read_op(cur.tb0, p0, 1, b1, 0, op_order(k >> 1), f0);
      });
      pw0 += 2048;
      pw1 += 2048;
      const uint32_t l0 = lbwB(b0);
      step(f0, nv_tag, [&](int k) __attribute__((always_inline)) {
        if ((k & 1) == 0) read_op(cur.tb0, p0, 1, b1, 1, op_order(k >> 1), f1);
        else if ((k & 3) == 1) issue_b(pw0, pw1, l0, k >> 2);
      });
      __builtin_amdgcn_s_waitcnt(vmcnt_only(8));
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
      __builtin_amdgcn_s_barrier();
      const uint32_t la = lbwA(p0);
      step(f1, nv_tag, [&](int k) __attribute__((always_inline)) {
        if ((k & 1) == 0) read_op(cur.tb0, p0 ^ 1, 0, b2, 0, op_order(k >> 1), f0);
        else issue_a(pa, cur.a_off, la, k >> 1);
      });
      pa += 128;
      pw0 += 2048;
      pw1 += 2048;
    };

    // the K loop, one copy per count of live token blocks (a ragged last row
    // block of an expert has fewer): the first two stages (their waits count
    // the previous tile's stores) and the last four (the next tile's loads)
    // take the general body, the others the fast one
    auto k_loop = [&](auto nv_tag) __attribute__((always_inline)) {
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      stage(0, P0{}, nv_tag);
      stage(1, P1{}, nv_tag);
      const unsigned char* pa = uni(cur.a + 128 * 3);
      const unsigned char* pw0 = uni(cur.w[0] + 2048 * 5);
      const unsigned char* pw1 = uni(cur.w[1] + 2048 * 5);
      for (int x = 2; x < nkb - kLNS; x += 2) fast(x, pa, pw0, pw1, nv_tag);
      stage(nkb - 4, P0{}, nv_tag);
      stage(nkb - 3, P1{}, nv_tag);
      stage(nkb - 2, P0{}, nv_tag);
      stage(nkb - 1, P1{}, nv_tag);
    };
    // ---- epilogue: round, pack and store.  Lane l holds token l mod 32 of a
    // block and columns 8q + 4 (l / 32) + 0..3 (q = 0..3) of a 32-column
    // block; one lane-pair swap gives lane l columns 16p + 0..7 and lane l + 32
    // columns 16p + 8..15.  Stored that way, a 16-byte-per-lane store writes 32
    // bytes into each of 32 rows, and the L2 takes 32 partial-line writes per
    // store (measured: the down kernel's stores cost it a quarter of its time
    // on the long prefill).  So each 32-row x 64-column piece (4 KB) goes
    // through LDS: the lanes write their chunks row-major (16-byte chunks
    // XOR-swizzled by row / 2, conflict-free both ways), read back 8 rows x 128
    // bytes per store, and each store writes 8 whole 128-byte row segments.
    // The staging area is this wave's 4 KB of the weight half of the tile's
    // last ring buffer: every wave has read that stage before the barrier of
    // the tile's last stage, and the next load into it is this wave's own (the
    // next tile's stage 0 issues it, after the wait at the end of here).  A
    // wave with NV < 4 live blocks rewrites its first block's outputs in the
    // slots of the others (same addresses, same bits), so every wave issues the
    // same number of stores.
    auto epilogue = [&](auto nv_tag) __attribute__((always_inline)) {
      constexpr int NV = decltype(nv_tag)::value;
      constexpr int kHalves = kJ / 2;                // 64-column pieces of the wave's columns
      const LTile& o = cur;
      unsigned char* stg = smem + kLBOff + ((ring + nkb - 1) & (kLNS - 1)) * kLStageB + wave * 4096;
      u32x4 first[NV < 4 ? kHalves : 1][4];
      typedef __attribute__((address_space(1))) unsigned char gbyte;
      typedef __attribute__((address_space(1))) u32x4 gu32x4;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int tb = m == 0 ? o.tb0 : 2 * m + wr;
        const bool live = m < NV;
#pragma unroll
        for (int hc = 0; hc < kHalves; ++hc) {
          u32x4 out4[4];
          if (live) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const int j = 2 * hc + jj;
              // read this block's accumulators only now: without the (empty)
              // asm the compiler copies every accumulator out of the AGPRs at
              // once and spills to make room
              asm volatile("" : "+a"(acc[m][j]));
              if constexpr (MODE == kGateUp) asm volatile("" : "+a"(acc[m][j + 2]));
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                uint32_t w[2][2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const int q = 2 * p + h;
                  float y[4];
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    if constexpr (MODE == kGateUp) {
                      const float gv = acc[m][j][4 * q + e], uv = acc[m][j + 2][4 * q + e];
                      y[e] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                    } else {
                      y[e] = acc[m][j][4 * q + e];
                    }
                  }
                  w[h][0] = pack_bf16x2(y[0], y[1]);
                  w[h][1] = pack_bf16x2(y[2], y[3]);
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                  const auto sw = __builtin_amdgcn_permlane32_swap(w[0][c], w[1][c], false, false);
                  w[0][c] = sw[0];
                  w[1][c] = sw[1];
                }
                // chunk c of row r (columns 8c .. 8c + 7 of the piece)
                const int r = lane & 31, c = 4 * jj + 2 * p + (lane >> 5);
                *reinterpret_cast<u32x4*>(stg + r * 128 + ((c ^ ((r >> 1) & 7)) << 4)) =
                    u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
              }
            }
#pragma unroll
            for (int sidx = 0; sidx < 4; ++sidx) {
              const int r = 8 * sidx + (lane >> 3), c = lane & 7;
              out4[sidx] = *reinterpret_cast<const u32x4*>(stg + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
              if constexpr (NV < 4) {
                if (m == 0) first[hc][sidx] = out4[sidx];
              }
            }
          } else {
#pragma unroll
            for (int sidx = 0; sidx < 4; ++sidx) {
              if constexpr (NV < 4) out4[sidx] = first[hc][sidx];
            }
          }
          // store sidx: rows 8 sidx + lane / 8 of the block, columns 64 hc +
          // 8 (lane mod 8) .. + 7; a global store (not flat: a flat store
          // would also count in lgkmcnt, which the next stages' LDS waits use)
#pragma unroll
          for (int sidx = 0; sidx < 4; ++sidx) {
            const int row = min(32 * (live ? tb : o.tb0) + 8 * sidx + (lane >> 3), o.valid - 1);
            const uint32_t off = (static_cast<uint32_t>(row) * static_cast<uint32_t>(o.ld) +
                                  static_cast<uint32_t>(64 * hc + 8 * (lane & 7))) * 2u;
            // down's outputs are non-temporal: the combine reads them once,
            // later, and left in L2 / MALL they would be written back to HBM
            // while it runs (long prefill: combine 253 -> 231 us, down 2%
            // faster); whole 128-byte segments, so nothing needs merging
            if constexpr (MODE == kDown) __builtin_nontemporal_store(out4[sidx], (gu32x4*)((gbyte*)o.out + off));
            else *(gu32x4*)((gbyte*)o.out + off) = out4[sidx];
          }
          // a few accumulators at a time
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the staging reads are done before this wave's next load into the area
      __builtin_amdgcn_s_waitcnt(lgkmcnt_only(0));
    };

    switch (nv) {
      case 4: k_loop(std::integral_constant<int, 4>{}); epilogue(std::integral_constant<int, 4>{}); break;
      case 3: k_loop(std::integral_constant<int, 3>{}); epilogue(std::integral_constant<int, 3>{}); break;
      case 2: k_loop(std::integral_constant<int, 2>{}); epilogue(std::integral_constant<int, 2>{}); break;
      default: k_loop(std::integral_constant<int, 1>{}); epilogue(std::integral_constant<int, 1>{}); break;
    }

    stored = true;
    ring = (ring + nkb) & (kLNS - 1);
    aring = (aring + (nkb >> 1)) & 1;
    ++round;
    ti = tn;
    if (has_next) cur = nxt;
  }
  // the last tile's trailing loads (repeats of its first stages) land in LDS
  // before the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

}  // namespace

bool lds_gemm_fits(int mode, const GemmArgs& a) {
  const int cols = mode == kGateUp ? kLBN / 2 : kLBN;
  if (a.E > kGemmMaxE) return false;
  if (a.E > 0 && (a.K % (2 * kLBK) != 0 || a.K < 8 * kLBK || a.N % cols != 0)) return false;
  if (a.has_shared && (a.Ks % (2 * kLBK) != 0 || a.Ks < 8 * kLBK || a.Ns % cols != 0)) return false;
  return true;
}

hipError_t launch_lds_gemm(int mode, const GemmArgs& a, hipStream_t st) {
  if (mode == kGateUp)
    lds_gemm_kernel<kGateUp><<<persistent_grid(), kLThreads, 0, st>>>(a);
  else
    lds_gemm_kernel<kDown><<<persistent_grid(), kLThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
