// Grouped GEMMs of the routed experts and the shared expert, bf16 operands on
// gfx950 MFMA with fp32 accumulation (FP8 weights are widened to bf16 in
// registers and their row scales applied to the accumulators).
//
// What they compute ("Laguna-M.1-base", Feed-forward: SwiGLU without biases;
// grouped GEMM over tokens in expert order, "Laguna M.1/XS.2 Technical Report",
// Key claims, report section 3.1.2):
//   gate_up  h[p]  = silu(Wg_e a_p) * (Wu_e a_p)   for the rows p of expert e,
//            and the shared expert over all tokens as one more group;
//   down     y[p]  = Wd_e h[p].
//
// Design (MI355X-first, not the pages' CUTLASS kernel):
//   * persistent grid: every workgroup derives the tile table from `offsets`
//     in LDS (tiles per group, inclusive scan), so no host synchronisation and
//     no extra launch are needed for ragged expert sizes;
//   * tile order: m-tiles of the same (group, n-tile) are adjacent; tiles go
//     out in rounds of one per workgroup, and each round is cut into 8 runs
//     of consecutive tiles, one per XCD (workgroup b runs on XCD b % 8), so
//     the workgroups that share a weight tile run at the same time behind the
//     same L2, and every workgroup gets the same number of tiles to within
//     one; the shared expert's row-block height is picked so that its tiles
//     fill the last round (gate_up spreads them through all rounds instead);
//   * tiles of BM token rows x 256 or 512 weight rows (BM by the mean rows per
//     expert, so an expert's rows mostly fit one tile and its weights stream
//     once), one workgroup per CU; weights, packed in MFMA fragment order,
//     stream from HBM straight into registers through a deep prefetch ring,
//     token rows go through an LDS ring (mma_stream.h); gate_up tiles pair each
//     gate block with the up block of the same columns, so SwiGLU is applied in
//     registers before one rounding to bf16;
//   * a tile's outputs are stored while the next tile's loads stream (see the
//     epilogue), a token block at a time through a small LDS staging area so
//     that each 16-byte-per-lane store writes whole row segments.
#include "grouped_gemm.h"
#include "mma_stream.h"

namespace moe {
namespace {

constexpr int kThreads = kPipeThreads;
constexpr int kMaxE = kGemmMaxE;
constexpr int kXcds = kGemmXcds;

// Output side of one tile.
template <int NB>
struct TileOut {
  bf16_t* out;      // element (row r of the tile, column c of the wave's) at out + r * ld + c
  int ld;
  int valid;        // rows of the tile that hold tokens
  const float* scale[NB];   // FP8 weights: the row scales of the wave's weight blocks
};

// One kernel for both GEMMs: a tile is BM token rows of one group x 256 weight
// rows (gate_up: 128 gate rows and the 128 up rows of the same columns; down:
// 256 output columns), computed by the weight-streaming pipeline
// (mma_stream.h).  Wave w holds the gate block and the up block of the same 32
// columns, so SwiGLU is applied in registers; outputs are rounded in registers
// and leave through a per-wave LDS staging area as whole row segments.
template <int MODE, int BM, int NB, int PF, bool W8>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs g) {
  using ST = StreamTile<BM, NB, PF, W8>;
  using TileOut = moe::TileOut<NB>;
  constexpr int MBW = ST::MBW;
  // output columns per tile: gate_up pairs NB / 2 gate blocks with the up
  // blocks of the same columns (32 NB / 2 columns per wave); down: 32 NB per wave
  constexpr int kWaveCols = (MODE == kGateUp) ? 16 * NB : 32 * NB;
  constexpr int kOutCols = 4 * kWaveCols;
  __shared__ __attribute__((aligned(16))) bf16_t lds[kStreamNS * ST::kAElems];
  // output staging: per wave one token block of its row segments (32 rows x
  // kRowB bytes), see store_block below
  constexpr int kRowB = kWaveCols * 2;
  __shared__ __attribute__((aligned(16))) unsigned char stg_all[4][32 * kRowB];
  static_assert(kStreamNS * ST::kAElems * 2 + 4 * 32 * kRowB + 2 * (kMaxE + 1) * 4 <= 160 * 1024, "LDS");
  __shared__ int tile_end[kMaxE + 1];
  __shared__ int row_base[kMaxE + 1];
  __shared__ int shared_bm;

  const int tid = threadIdx.x;
  const int E = g.E;
  const int nt_r = g.N / kOutCols;
  const int nt_s = g.has_shared ? g.Ns / kOutCols : 0;
  const int G = gridDim.x;                 // workgroups, a multiple of kXcds

  // ---- tile table: tiles per routed group, inclusive scan, shared group last
  {
    int cnt = 0;
    if (tid < E) {
      // clamped so that no offsets table can move a tile outside [0, S)
      const int lo = min(max(g.offsets[tid], 0), g.S);
      const int hi = min(max(g.offsets[tid + 1], lo), g.S);
      row_base[tid] = lo;
      cnt = ((hi - lo) + BM - 1) / BM * nt_r;
    }
    // inclusive scan: within each wave by lane shuffles, then the totals of
    // the waves before (two barriers instead of one pair per doubling step)
    const int ln = tid & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(cnt, d);
      if (ln >= d) cnt += v;
    }
    if (ln == 63) tile_end[tid] = cnt;                 // the wave's total, at its last entry
    __syncthreads();
    for (int w = 0; w < (tid >> 6); ++w) cnt += tile_end[64 * w + 63];
    __syncthreads();
    tile_end[tid] = cnt;
    __syncthreads();
    if (tid == 0) {
      const int routed_total = E > 0 ? tile_end[E - 1] : 0;
      // Shared-expert row-block height: the tiles run in rounds of G (one per
      // workgroup), routed tiles first, so the shared tiles fill the last
      // rounds.  Take the fewest rounds, and for that count the shortest
      // blocks: the shared weights are read by every block of a round from
      // L2, and shorter blocks spread them evenly over the workgroups.
      int best_bm = BM, best_rounds = 0x7fffffff;
      if (g.has_shared) {
        for (int bm = 32; bm <= BM; bm += 32) {
          const int rounds = (routed_total + (g.T + bm - 1) / bm * nt_s + G - 1) / G;
          if (rounds < best_rounds) {
            best_rounds = rounds;
            best_bm = bm;
          }
        }
      }
      shared_bm = best_bm;
      tile_end[E] = routed_total + (g.has_shared ? (g.T + best_bm - 1) / best_bm * nt_s : 0);
      row_base[E] = E > 0 ? min(max(g.offsets[E], row_base[E - 1]), g.S) : 0;
    }
    __syncthreads();
  }
  const int total = __builtin_amdgcn_readfirstlane(tile_end[E]);
  const int sbm = __builtin_amdgcn_readfirstlane(shared_bm);

  // ---- XCD-aware persistent assignment: tiles go out in rounds of G; each
  // round is cut into 8 runs of G / 8 consecutive tiles, one per XCD
  // (workgroup b runs on XCD b % 8 and takes the (b / 8)-th tile of its XCD's
  // run), so the workgroups that read the same weights -- the row blocks of
  // one expert and column block -- run at the same time behind the same L2,
  // and no workgroup gets more than one tile more than another.  Cut that way
  // a partial last round leaves the last XCDs idle; when it is a large share
  // of the work (at most 5 rounds: decode-sized batches) it is split evenly
  // over the 8 XCDs instead (measured: 2% off the decode GEMMs; on the long
  // M.1-width launches the even split cost 2%).
  const int xcd = blockIdx.x % kXcds, in_xcd = blockIdx.x / kXcds;
  const bool even_last = total <= 5 * G;
  auto tile_at = [&](int r) -> int {      // this workgroup's tile of round r, or -1
    const int base = r * G;
    if (base >= total) return -1;
    const int n = min(G, total - base);
    if (n == G || !even_last) {
      const int t = xcd * (G / kXcds) + in_xcd;
      return t < n ? base + t : -1;
    }
    const int q = n / kXcds, rem = n % kXcds;
    if (in_xcd >= q + (xcd < rem ? 1 : 0)) return -1;
    return base + xcd * q + min(xcd, rem) + in_xcd;
  };
  const int pos = tile_at(0);
  if (pos < 0) return;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // ---- sources and output of tile ti (all but the token-row offsets uniform)
  auto decode = [&](int ti, StreamSrc<BM, NB>& src, TileOut& o) {
    // per-lane row / column arithmetic is redone here for every tile: hoisted
    // out of the tile loop it would hold registers across the whole stream
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    if (g.spread_shared && E > 0) {
      // gate_up: the shared expert's tiles (weights L2-resident after the
      // first few) are spread evenly through the schedule instead of filling
      // the last round, so that every round keeps most CUs on the HBM weight
      // stream: schedule slot ti holds shared tile c0 when floor((ti + 1) ns /
      // total) steps past c0 = floor(ti ns / total), else routed tile ti - c1
      const int routed_total = __builtin_amdgcn_readfirstlane(tile_end[E - 1]);
      const int ns = total - routed_total;
      const int c1 = static_cast<int>((static_cast<long long>(ti) + 1) * ns / total);
      const int c0 = static_cast<int>(static_cast<long long>(ti) * ns / total);
      ti = c1 > c0 ? routed_total + c0 : ti - c1;
    }
    int lo = 0, hi = E;                     // group: first with tile_end > ti
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tile_end[mid] > ti) hi = mid; else lo = mid + 1;
    }
    const int grp = __builtin_amdgcn_readfirstlane(lo);
    const bool shared = grp == E;
    const int first = grp == 0 ? 0 : __builtin_amdgcn_readfirstlane(tile_end[grp - 1]);
    const int rb = shared ? 0 : __builtin_amdgcn_readfirstlane(row_base[grp]);
    const int M = shared ? g.T : __builtin_amdgcn_readfirstlane(row_base[grp + 1]) - rb;
    const int bm = shared ? sbm : BM;       // row-block height of this group
    const int mt = (M + bm - 1) / bm;
    const int local = ti - first;
    const int m0 = (local % mt) * bm;
    const int n_tile = local / mt;
    const int K = shared ? g.Ks : g.K;
    const int Nout = shared ? g.Ns : g.N;
    const int n0 = n_tile * kOutCols;
    const int valid = min(bm, M - m0);
    src.nkb = K / kStreamBK;

    // token rows: lane's chunk of LDS load q is row 8 (MBW wave + q) + lane / 8
    // of the tile (rows past the tile's last one repeat it)
    const bool gathered = !shared && g.gather != nullptr;
    if (gathered) {
      src.a_base = g.a_routed;
    } else if (shared) {
      src.a_base = g.a_shared + static_cast<size_t>(m0) * K;
    } else {
      src.a_base = g.a_routed + static_cast<size_t>(rb + m0) * K;
    }
    // gathered rows: the token ids of the wave's 8 MBW consecutive rows come
    // in one window of scalar loads only (a vector load here would make the
    // compiler wait for the whole weight stream in flight); near the end of
    // the array the window's loads are clamped one by one.  Rows past the
    // tile's last take its last row's id, like the rows of the other modes,
    // so that their results equal that row's.
    const int wstart = rb + m0 + 8 * MBW * wave;
    int win[8 * MBW];
    int last_tok = 0;
    if (gathered) {
      const __attribute__((address_space(4))) int32_t* gt =
          (const __attribute__((address_space(4))) int32_t*)(g.gather);
      last_tok = gt[rb + m0 + valid - 1];
      if (wstart + 8 * MBW <= g.S) {
#pragma unroll
        for (int i = 0; i < 8 * MBW; ++i) win[i] = gt[wstart + i];
      } else {
#pragma unroll
        for (int i = 0; i < 8 * MBW; ++i) win[i] = gt[min(wstart + i, g.S - 1)];
      }
    }
#pragma unroll
    for (int q = 0; q < MBW; ++q) {
      int row, col;
      chunk_source(stream_a_slot<MBW>(q, wave, lane), row, col);
      uint32_t r;
      if (gathered) {
        int tok = win[8 * q];
#pragma unroll
        for (int i = 1; i < 8; ++i) tok = (lane >> 3) == i ? win[8 * q + i] : tok;
        tok = row < valid ? tok : last_tok;
        r = static_cast<uint32_t>(min(max(tok, 0), g.T - 1));
      } else {
        r = static_cast<uint32_t>(min(row, valid - 1));
      }
      src.a_off[q] = (r * static_cast<uint32_t>(K) + static_cast<uint32_t>(col)) * 2u;
    }
    // packed weights: the wave's 32-row blocks, 32 K bytes per row block and
    // element byte (1 for FP8 codes, 2 for bf16)
    constexpr int kWB = W8 ? 1 : 2;
    const int Nw = MODE == kGateUp ? 2 * Nout : Nout;             // rows of one weight matrix
    const unsigned char* wbase =
        shared ? g.w_shared : g.w_routed + static_cast<size_t>(grp) * Nw * K * kWB;
    const float* sbase = W8 ? (shared ? g.s_shared : g.s_routed + static_cast<size_t>(grp) * Nw) : nullptr;
    // the wave's weight block rows and its first output column
    const int col0 = n0 + kWaveCols * wave;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // gate_up: blocks j < NB / 2 are gate rows, the others the up rows of
      // the same columns; down: NB consecutive blocks
      const int wrow = MODE == kGateUp ? (j < NB / 2 ? col0 + 32 * j : Nout + col0 + 32 * (j - NB / 2))
                                       : col0 + 32 * j;
      src.w[j] = wbase + static_cast<size_t>(wrow >> 5) * K * 32 * kWB;
      o.scale[j] = W8 ? sbase + wrow : nullptr;
    }
    o.out = (shared ? g.out_shared + static_cast<size_t>(m0) * Nout
                    : g.out_routed + static_cast<size_t>(rb + m0) * Nout) + col0;
    o.ld = Nout;
    o.valid = valid;
  };

  StreamSrc<BM, NB> cur, nxt;
  TileOut ocur, onxt;
  StreamState<NB, PF> ss;
  // A tile's outputs are rounded and packed, 8 bf16 per lane and store.  With
  // 2 weight blocks per wave they wait in registers and are stored during the
  // next tile's last K blocks, a token block at a time among its loads: stored at the
  // tile's end they would queue behind the next tile's whole prefetch and
  // hold every wave up.  The 4-block shapes have no registers to spare and
  // store at the tile's end (the next tile's first waits count those stores).
  // Rows past the tile's last rewrite its last row, whose values they repeat
  // bit for bit, so the number of stores is a constant.
  //
  // A packed value (lane l: token l mod 32 of block m, 8 columns at 32 j +
  // 16 p + 8 (l / 32)) stored as it is writes 32 bytes into each of 32 rows: 32
  // partial-line writes for the L2 per store, which measured as a large share
  // of these kernels' time at the XS.2 shape.  So a block's values go through
  // this wave's staging area in LDS: written row-major (16-byte chunks
  // XOR-swizzled, conflict-free for the column-wise writes and the row-wise
  // reads), read back as whole row segments (kRowB bytes per row: 64, 128 or
  // 256), 1 KB per store, as many stores as before.
  constexpr int kJ = MODE == kGateUp ? NB / 2 : NB;   // output blocks of 32 columns per wave
  constexpr int kStores = MBW * kJ * 2;
  constexpr bool kDefer = NB == 2;
  constexpr int kChunks = kRowB / 16;                 // 16-byte chunks per row segment (4 kJ)
  constexpr int kSwzShift = kRowB == 64 ? 2 : (kRowB == 128 ? 1 : 0);
  static_assert(kChunks == 4 * kJ && (kRowB == 64 || kRowB == 128 || kRowB == 256), "row segments");
  typedef __attribute__((address_space(1))) unsigned char gbyte;
  typedef __attribute__((address_space(1))) u32x4 gu32x4;
  unsigned char* stg = stg_all[__builtin_amdgcn_readfirstlane(tid >> 6)];
  auto chunk_at = [&](int r, int c) { return stg + r * kRowB + ((c ^ ((r >> kSwzShift) & (kChunks - 1))) << 4); };
  uint4 pend[kStores];
  TileOut opend;
  bool has_pend = false;
  // value (j, p) of block m into the staging area
  auto stage_value = [&](int j, int p, const uint4& v) {
    *reinterpret_cast<u32x4*>(chunk_at(lane & 31, 4 * j + 2 * p + (lane >> 5))) = u32x4{v.x, v.y, v.z, v.w};
  };
  // the staged block m of tile `o`, read back and stored: store s writes rows
  // s (64 / kChunks) + l / kChunks, chunk l mod kChunks
  auto store_staged = [&](int m, const TileOut& o) {
#pragma unroll
    for (int s_idx = 0; s_idx < 2 * kJ; ++s_idx) {
      const int r = s_idx * (64 / kChunks) + lane / kChunks, c = lane % kChunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(chunk_at(r, c));
      const int row = min(32 * m + r, o.valid - 1);
      const uint32_t off = (static_cast<uint32_t>(row) * static_cast<uint32_t>(o.ld) + 8u * c) * 2u;
      *(gu32x4*)((gbyte*)o.out + off) = v;
    }
  };
  auto store_block = [&](int m) {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) stage_value(j, p, pend[(m * kJ + j) * 2 + p]);
    store_staged(m, opend);
  };
  decode(pos, cur, ocur);
  stream_start<BM, NB, PF>(cur, ss, lds);
  int round = 0;
  for (int ti = pos; ti >= 0; ti = tile_at(++round)) {
    const TileOut o = ocur;
    f32x16 acc[MBW][NB];
    // FP8: the row scales of the lane's 16 accumulator rows per weight block,
    // loaded in the tile's last K blocks (ordinary loads: the epilogue's wait
    // for them counts the loads issued after them)
    float wsc[W8 ? NB : 1][16];
    stream_tile<BM, NB, PF, W8, kDefer ? 0 : kStores>(cur, nxt, [&]() {
      const int tn = tile_at(round + 1);
      if (tn < 0) return false;
      decode(tn, nxt, onxt);
      return true;
    }, [&](auto u_tag) {
      constexpr int u = decltype(u_tag)::value;
      if constexpr (W8 && u == 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // rows 8q + 4 (l / 32) + 0..3 of the block: registers 4q..4q+3
            const float4 v = *reinterpret_cast<const float4*>(o.scale[j] + 8 * q + 4 * (lane >> 5));
            wsc[j][4 * q] = v.x;
            wsc[j][4 * q + 1] = v.y;
            wsc[j][4 * q + 2] = v.z;
            wsc[j][4 * q + 3] = v.w;
          }
      }
      if (kDefer && has_pend) {
        // the previous tile's blocks, spread over the 4 tail blocks
#pragma unroll
        for (int m = MBW * u / 4; m < MBW * (u + 1) / 4; ++m) store_block(m);
      }
    }, ss, lds, acc, !kDefer && has_pend);
    // epilogue: round and pack.  Lane l holds columns 8q + 4 (l / 32) + 0..3
    // of its token for q = 0..3; one lane-pair swap (lanes l and l + 32) gives
    // lane l columns 16p + 0..7 and lane l + 32 columns 16p + 8..15.
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {          // registers 8p..8p+7: quads q = 2p, 2p + 1
          uint32_t v[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int q = 2 * p + h;
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (MODE == kGateUp) {
                float gv = acc[m][j][4 * q + e], uv = acc[m][j + NB / 2][4 * q + e];
                if constexpr (W8) {
                  gv *= wsc[j][4 * q + e];
                  uv *= wsc[j + NB / 2][4 * q + e];
                }
                y[e] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
              } else {
                y[e] = acc[m][j][4 * q + e];
                if constexpr (W8) y[e] *= wsc[j][4 * q + e];
              }
            }
            v[h][0] = pack_bf16x2(y[0], y[1]);
            v[h][1] = pack_bf16x2(y[2], y[3]);
          }
          // lanes < 32 keep quad 2p and take the upper lanes' quad 2p; lanes
          // >= 32 take the lower lanes' quad 2p + 1 and keep theirs
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const auto sw = __builtin_amdgcn_permlane32_swap(v[0][c], v[1][c], false, false);
            v[0][c] = sw[0];
            v[1][c] = sw[1];
          }
          const uint4 val = make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
          if constexpr (kDefer) {
            pend[(m * kJ + j) * 2 + p] = val;
          } else {
            stage_value(j, p, val);
            // a few accumulators at a time: reading them all out at once
            // would need as many VGPRs, on top of the weight ring in flight
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (!kDefer) store_staged(m, o);
    }
    opend = o;
    has_pend = true;
    cur = nxt;
    ocur = onxt;
  }
  // the last tile's outputs
  if (kDefer) {
#pragma unroll
    for (int m = 0; m < MBW; ++m) store_block(m);
  }
  stream_finish();
}


// Tile shape by the mean rows per expert (k*T/E).  Up to ~200 rows the weight
// stream from HBM is the limit: tall row blocks (an expert's rows mostly fit
// one, so its weights stream once), 2 weight blocks per wave and a deep weight
// prefetch (16 steps); shorter blocks for decode-sized batches.  Beyond that
// MFMA issue, LDS reads and the L2 traffic of re-read weights compete: 96-row
// blocks with 4 weight blocks per wave (each A fragment read from LDS feeds 4
// MFMAs) measured best among the shapes whose accumulators and weight ring fit
// the registers, when the output width allows their wider tiles.
template <int MODE, bool W8>
hipError_t launch_tiles(const GemmArgs& a, int mean_rows, hipStream_t st) {
  // the weight ring's depth: 16 K steps of bf16 weights, 8 ring steps (16 K
  // steps) of FP8 ones
  constexpr int P = W8 ? 8 : 16;
  const int wide = MODE == kGateUp ? 256 : 512;            // output columns of an NB = 4 tile
  // The LDS-tiled kernel (256 x 256 tiles, both operands through LDS) beats
  // the weight-streaming tiles below once an expert has a full 256-row tile
  // on average.  Measured (D = 4096, F = 1024 and D = 2048, F = 512): down
  // 7-11% faster at 256, 512 and 1024 rows per expert; gate/up 3% faster at
  // 256 and 512, 11% at 1024
  const int lds_from = 256;
  if (!W8 && mean_rows >= lds_from && lds_gemm_fits(MODE, a)) return launch_lds_gemm(MODE, a, st);
  if (mean_rows >= 192 && a.N % wide == 0 && (!a.has_shared || a.Ns % wide == 0))
    grouped_gemm_kernel<MODE, 96, 4, 8, W8><<<persistent_grid(), kThreads, 0, st>>>(a);
  else if (mean_rows >= 96)
    grouped_gemm_kernel<MODE, 160, 2, P, W8><<<persistent_grid(), kThreads, 0, st>>>(a);
  else if (mean_rows >= 48)
    grouped_gemm_kernel<MODE, 128, 2, P, W8><<<persistent_grid(), kThreads, 0, st>>>(a);
  else if (mean_rows >= 24)
    grouped_gemm_kernel<MODE, 64, 2, P, W8><<<persistent_grid(), kThreads, 0, st>>>(a);
  else
    grouped_gemm_kernel<MODE, 32, 2, P, W8><<<persistent_grid(), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

int mean_rows(const moe_shape& s) { return (s.T * s.k) / s.E; }

GemmArgs gate_up_args(const moe_shape& s, const bf16_t* x_perm, const int32_t* sorted_token,
                      const bf16_t* x, const int32_t* offsets, bf16_t* h) {
  GemmArgs a{};
  a.a_routed = x_perm ? x_perm : x;
  a.gather = x_perm ? nullptr : sorted_token;
  a.a_shared = x;
  a.out_routed = h;
  a.out_shared = h + static_cast<size_t>(s.T) * s.k * s.F;
  a.offsets = offsets;
  a.T = s.T;
  a.E = s.E;
  a.S = s.T * s.k;
  a.K = s.D;
  a.Ks = s.D;
  a.N = s.F;
  a.Ns = s.Fs;
  a.has_shared = s.Fs > 0;
  a.spread_shared = 1;
  return a;
}

GemmArgs down_args(const moe_shape& s, const bf16_t* h, const int32_t* offsets, bf16_t* y_perm,
                   bf16_t* y_shared) {
  GemmArgs a{};
  a.a_routed = h;
  a.gather = nullptr;
  a.a_shared = h + static_cast<size_t>(s.T) * s.k * s.F;
  a.out_routed = y_perm;
  a.out_shared = y_shared;
  a.offsets = offsets;
  a.T = s.T;
  a.E = s.E;
  a.S = s.T * s.k;
  a.K = s.F;
  a.Ks = s.Fs;
  a.N = s.D;
  a.Ns = s.D;
  a.has_shared = s.Fs > 0;
  return a;
}

}  // namespace

int persistent_grid() {
  static int grid = 0;
  if (grid == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      hipDeviceProp_t p;
      if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
        cus = p.multiProcessorCount;
    }
    grid = ((cus + kXcds - 1) / kXcds) * kXcds;   // one workgroup per CU
  }
  return grid;
}

// ---- training pass: the same kernel in its plain mode (no SwiGLU) on other
// operands.  Packed transposed weights (moe_pack_weights_transposed) turn the
// backward products into the forward's form: rows of the packed matrix are
// output columns, its K the reduction.

hipError_t launch_gate_up_pre_bf16(const moe_shape& s, const bf16_t* x_perm,
                                   const int32_t* sorted_token, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* wgu, const bf16_t* wsgu,
                                   bf16_t* gu, hipStream_t st) {
  // [g | u] = a [W_g; W_u]^T: the gate/up matrix read as one [2F, D] matrix
  GemmArgs a = gate_up_args(s, x_perm, sorted_token, x, offsets, gu);
  a.out_shared = gu + static_cast<size_t>(s.T) * s.k * 2 * s.F;
  a.N = 2 * s.F;
  a.Ns = 2 * s.Fs;
  a.w_routed = reinterpret_cast<const unsigned char*>(wgu);
  a.w_shared = reinterpret_cast<const unsigned char*>(wsgu);
  return launch_tiles<kDown, false>(a, mean_rows(s), st);
}

hipError_t launch_dgrad_h_bf16(const moe_shape& s, const bf16_t* dy_perm, const bf16_t* dout,
                               const int32_t* offsets, const bf16_t* wd_t, const bf16_t* wsd_t,
                               bf16_t* dh, hipStream_t st) {
  // dh = dy W_d: rows of W_d^T [F, D] are the outputs, D the reduction; the
  // shared expert's output gradient is dout itself
  GemmArgs a{};
  a.a_routed = dy_perm;
  a.a_shared = dout;
  a.out_routed = dh;
  a.out_shared = dh + static_cast<size_t>(s.T) * s.k * s.F;
  a.offsets = offsets;
  a.T = s.T;
  a.E = s.E;
  a.S = s.T * s.k;
  a.K = s.D;
  a.Ks = s.D;
  a.N = s.F;
  a.Ns = s.Fs;
  a.has_shared = s.Fs > 0;
  a.spread_shared = 1;
  a.w_routed = reinterpret_cast<const unsigned char*>(wd_t);
  a.w_shared = reinterpret_cast<const unsigned char*>(wsd_t);
  return launch_tiles<kDown, false>(a, mean_rows(s), st);
}

hipError_t launch_dgrad_x_bf16(const moe_shape& s, const bf16_t* dgu, const int32_t* offsets,
                               const bf16_t* wgu_t, const bf16_t* wsgu_t, bf16_t* dx_perm,
                               bf16_t* dx_shared, hipStream_t st) {
  // da = [dg | du] [W_g; W_u]: rows of the transposed gate/up matrix [D, 2F]
  GemmArgs a{};
  a.a_routed = dgu;
  a.a_shared = dgu + static_cast<size_t>(s.T) * s.k * 2 * s.F;
  a.out_routed = dx_perm;
  a.out_shared = dx_shared;
  a.offsets = offsets;
  a.T = s.T;
  a.E = s.E;
  a.S = s.T * s.k;
  a.K = 2 * s.F;
  a.Ks = 2 * s.Fs;
  a.N = s.D;
  a.Ns = s.D;
  a.has_shared = s.Fs > 0;
  a.spread_shared = 1;
  a.w_routed = reinterpret_cast<const unsigned char*>(wgu_t);
  a.w_shared = reinterpret_cast<const unsigned char*>(wsgu_t);
  return launch_tiles<kDown, false>(a, mean_rows(s), st);
}

hipError_t launch_dense_bf16(int rows, int K, int N, const bf16_t* a_rows, const bf16_t* w_packed,
                             bf16_t* out, hipStream_t st) {
  // out [rows, N] = a [rows, K] W^T with W packed [N, K]: the shared group
  // alone, no routed groups
  GemmArgs a{};
  a.a_shared = a_rows;
  a.w_shared = reinterpret_cast<const unsigned char*>(w_packed);
  a.out_shared = out;
  a.T = rows;
  a.E = 0;
  a.S = 0;
  a.Ks = K;
  a.Ns = N;
  a.has_shared = 1;
  return launch_tiles<kDown, false>(a, rows, st);
}

hipError_t launch_gate_up_bf16(const moe_shape& s, const bf16_t* x_perm,
                               const int32_t* sorted_token, const bf16_t* x,
                               const int32_t* offsets, const bf16_t* wgu, const bf16_t* wsgu,
                               bf16_t* h, hipStream_t st) {
  GemmArgs a = gate_up_args(s, x_perm, sorted_token, x, offsets, h);
  a.w_routed = reinterpret_cast<const unsigned char*>(wgu);
  a.w_shared = reinterpret_cast<const unsigned char*>(wsgu);
  a.has_shared = a.has_shared && wsgu != nullptr;     // no shared weights: routed experts only
  return launch_tiles<kGateUp, false>(a, mean_rows(s), st);
}

hipError_t launch_down_bf16(const moe_shape& s, const bf16_t* h, const int32_t* offsets,
                            const bf16_t* wd, const bf16_t* wsd, bf16_t* y_perm,
                            bf16_t* y_shared, hipStream_t st) {
  GemmArgs a = down_args(s, h, offsets, y_perm, y_shared);
  a.w_routed = reinterpret_cast<const unsigned char*>(wd);
  a.w_shared = reinterpret_cast<const unsigned char*>(wsd);
  a.has_shared = a.has_shared && wsd != nullptr;      // no shared weights: routed experts only
  return launch_tiles<kDown, false>(a, mean_rows(s), st);
}

hipError_t launch_shared_ffn_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wsgu,
                                  const bf16_t* wsd, bf16_t* hs, bf16_t* ys, hipStream_t st) {
  // the shared expert alone: both GEMMs with the shared group only (E = 0)
  GemmArgs a{};
  a.a_shared = x;
  a.w_shared = reinterpret_cast<const unsigned char*>(wsgu);
  a.out_shared = hs;
  a.T = s.T;
  a.Ks = s.D;
  a.Ns = s.Fs;
  a.has_shared = 1;
  if (hipError_t e = launch_tiles<kGateUp, false>(a, s.T, st)) return e;
  GemmArgs b{};
  b.a_shared = hs;
  b.w_shared = reinterpret_cast<const unsigned char*>(wsd);
  b.out_shared = ys;
  b.T = s.T;
  b.Ks = s.Fs;
  b.Ns = s.D;
  b.has_shared = 1;
  return launch_tiles<kDown, false>(b, s.T, st);
}

hipError_t launch_gate_up_fp8(const moe_shape& s, const bf16_t* x_perm, const int32_t* sorted_token,
                              const bf16_t* x, const int32_t* offsets, const uint8_t* wgu,
                              const float* sgu, const uint8_t* wsgu, const float* ssgu, bf16_t* h,
                              hipStream_t st) {
  GemmArgs a = gate_up_args(s, x_perm, sorted_token, x, offsets, h);
  a.w_routed = wgu;
  a.w_shared = wsgu;
  a.s_routed = sgu;
  a.s_shared = ssgu;
  return launch_tiles<kGateUp, true>(a, mean_rows(s), st);
}

hipError_t launch_down_fp8(const moe_shape& s, const bf16_t* h, const int32_t* offsets,
                           const uint8_t* wd, const float* sd, const uint8_t* wsd, const float* ssd,
                           bf16_t* y_perm, bf16_t* y_shared, hipStream_t st) {
  GemmArgs a = down_args(s, h, offsets, y_perm, y_shared);
  a.w_routed = wd;
  a.w_shared = wsd;
  a.s_routed = sd;
  a.s_shared = ssd;
  return launch_tiles<kDown, true>(a, mean_rows(s), st);
}

}  // namespace moe
