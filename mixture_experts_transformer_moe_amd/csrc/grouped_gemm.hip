// Grouped GEMMs of the routed experts and the shared expert, bf16 operands on
// gfx950 MFMA with fp32 accumulation.
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
//   * tile order: m-tiles of the same (group, n-tile) are adjacent, and the
//     tile range is cut into 8 contiguous chunks, one per XCD (workgroup b runs
//     on XCD b % 8), so the workgroups that share a weight tile run at the
//     same time behind the same L2;
//   * 128 x 128 x 64 block tile, 4 waves of 64 x 64, v_mfma_f32_32x32x16_bf16,
//     double-buffered LDS with an XOR swizzle of the 16-byte chunks (conflict-
//     free ds_read_b128), global loads for step k+1 in flight during step k;
//   * gate_up: the 128 B-rows of a tile are 64 gate rows and the 64 matching up
//     rows, and every wave holds a gate block and the up block of the same
//     columns, so SwiGLU is applied in registers before one rounding to bf16;
//   * epilogue staged through LDS for 16-byte coalesced row stores.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;           // B rows per tile
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kMaxE = 256;
constexpr int kXcds = 8;

enum Mode { kGateUp = 0, kDown = 1 };

struct GemmArgs {
  const bf16_t* a_routed;   // [S, K] rows in expert order (x_perm or h), or x when gather != null
  const int32_t* gather;    // sorted_token (A row p = x[gather[p]]) or null
  const bf16_t* a_shared;   // [T, Ks]
  const bf16_t* w_routed;   // [E, Nw, K]
  const bf16_t* w_shared;   // [Nws, Ks]
  bf16_t* out_routed;       // [S, N]
  bf16_t* out_shared;       // [T, Ns]
  const int32_t* offsets;   // [E + 1]
  int T, E, S;
  int K, Ks;                // reduction length (routed / shared)
  int N, Ns;                // output columns (routed / shared)
  int has_shared;
};

// element offset of 16-byte chunk `ch` of row `row` in a [rows][64] bf16 tile
__device__ __forceinline__ int swz(int row, int ch) { return row * BK + ((ch ^ (row & 7)) << 3); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(GemmArgs g) {
  constexpr int kOutCols = (MODE == kGateUp) ? BN / 2 : BN;   // output columns per tile
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * BK];
  __shared__ int tile_end[kMaxE + 1];
  __shared__ int row_base[kMaxE + 1];

  const int tid = threadIdx.x;
  const int E = g.E;
  const int nt_r = g.N / kOutCols;
  const int nt_s = g.has_shared ? g.Ns / kOutCols : 0;

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
    tile_end[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kMaxE; off <<= 1) {
      const int v = tid >= off ? tile_end[tid - off] : 0;
      __syncthreads();
      tile_end[tid] += v;
      __syncthreads();
    }
    if (tid == 0) {
      const int routed_total = tile_end[E - 1];
      tile_end[E] = routed_total + (g.has_shared ? (g.T + BM - 1) / BM * nt_s : 0);
      row_base[E] = min(max(g.offsets[E], row_base[E - 1]), g.S);
    }
    __syncthreads();
  }
  const int total = tile_end[E];

  // ---- XCD-aware persistent assignment
  const int P = gridDim.x;                 // multiple of kXcds
  const int per_xcd = P / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int t_lo = xcd * chunk;
  const int t_hi = min(total, t_lo + chunk);

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  for (int ti = t_lo + slot; ti < t_hi; ti += per_xcd) {
    // group of this tile: first g with tile_end[g] > ti
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tile_end[mid] > ti) hi = mid; else lo = mid + 1;
    }
    const int grp = lo;
    const bool shared = grp == E;
    const int first = grp == 0 ? 0 : tile_end[grp - 1];
    const int M = shared ? g.T : row_base[grp + 1] - row_base[grp];
    const int mt = (M + BM - 1) / BM;
    const int local = ti - first;
    const int m0 = (local % mt) * BM;
    const int n_tile = local / mt;
    const int K = shared ? g.Ks : g.K;
    const int Nout = shared ? g.Ns : g.N;
    const int KT = K / BK;

    // ---- per-thread source rows for the A and B tiles (4 chunks each)
    const bf16_t* a_ptr[4];
    const bf16_t* b_ptr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + kThreads * q;
      const int row = c >> 3, ch = c & 7;
      const int r = min(m0 + row, M - 1);                // rows past M are computed and dropped
      const bf16_t* arow;
      if (shared) {
        arow = g.a_shared + static_cast<size_t>(r) * K;
      } else if (g.gather) {
        const int t = min(max(g.gather[row_base[grp] + r], 0), g.T - 1);
        arow = g.a_routed + static_cast<size_t>(t) * K;
      } else {
        arow = g.a_routed + static_cast<size_t>(row_base[grp] + r) * K;
      }
      a_ptr[q] = arow + ch * 8;
      int wrow;
      if (MODE == kGateUp) {
        const int n0 = n_tile * kOutCols;
        wrow = row < kOutCols ? n0 + row : Nout + n0 + (row - kOutCols);
      } else {
        wrow = n_tile * BN + row;
      }
      const bf16_t* wbase = shared ? g.w_shared
                                   : g.w_routed + static_cast<size_t>(grp) * (MODE == kGateUp ? 2 * Nout : Nout) * K;
      b_ptr[q] = wbase + static_cast<size_t>(wrow) * K + ch * 8;
    }

    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra[q] = *reinterpret_cast<const u32x4*>(a_ptr[q] + k0);
        rb[q] = *reinterpret_cast<const u32x4*>(b_ptr[q] + k0);
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + kThreads * q;
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(&lds[buf][swz(row, ch)]) = ra[q];
        *reinterpret_cast<u32x4*>(&lds[buf][BM * BK + swz(row, ch)]) = rb[q];
      }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0.f};

    // rows of this wave's MFMA blocks inside the tile
    int arow_blk[2], brow_blk[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) arow_blk[i] = 64 * wm + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      brow_blk[j] = (MODE == kGateUp ? 64 * j + 32 * wn : 64 * wn + 32 * j) + (lane & 31);
    const int khalf = lane >> 5;

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) gload((kt + 1) * BK);
      const bf16_t* As = &lds[buf][0];
      const bf16_t* Bs = &lds[buf][BM * BK];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = 2 * kk + khalf;
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&As[swz(arow_blk[i], ch)]));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Bs[swz(brow_blk[j], ch)]));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: registers -> LDS tile (bf16) -> 16-byte row stores
    bf16_t* stage = &lds[0][0];
    constexpr int kStageLd = kOutCols + 8;           // padded row (bf16 elements)
    // C layout: lane holds column (lane & 31), register r -> row (r/4)*8 + (lane/32)*4 + r%4
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 64 * wm + 32 * i + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (MODE == kGateUp) {
          const int col = 32 * wn + (lane & 31);
          const float gv = acc[i][0][r], uv = acc[i][1][r];
          stage[row * kStageLd + col] = f32_to_bf16(gv / (1.0f + __expf(-gv)) * uv);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = 64 * wn + 32 * j + (lane & 31);
            stage[row * kStageLd + col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    }
    __syncthreads();
    constexpr int kChunksPerRow = kOutCols / 8;
    bf16_t* out = shared ? g.out_shared : g.out_routed + static_cast<size_t>(row_base[grp]) * Nout;
    const int n0 = n_tile * kOutCols;
    for (int c = tid; c < BM * kChunksPerRow; c += kThreads) {
      const int row = c / kChunksPerRow, ch = c % kChunksPerRow;
      if (m0 + row < M) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[row * kStageLd + ch * 8]);
        *reinterpret_cast<u32x4*>(out + static_cast<size_t>(m0 + row) * Nout + n0 + ch * 8) = v;
      }
    }
    __syncthreads();
  }
}

int persistent_grid() {
  static int grid = 0;
  if (grid == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      hipDeviceProp_t p;
      if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
        cus = p.multiProcessorCount;
    }
    grid = ((cus * 2 + kXcds - 1) / kXcds) * kXcds;   // two workgroups per CU
  }
  return grid;
}

}  // namespace

hipError_t launch_gate_up_bf16(const moe_shape& s, const bf16_t* x_perm,
                               const int32_t* sorted_token, const bf16_t* x,
                               const int32_t* offsets, const bf16_t* wgu, const bf16_t* wsgu,
                               bf16_t* h, hipStream_t st) {
  GemmArgs a;
  a.a_routed = x_perm ? x_perm : x;
  a.gather = x_perm ? nullptr : sorted_token;
  a.a_shared = x;
  a.w_routed = wgu;
  a.w_shared = wsgu;
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
  grouped_gemm_kernel<kGateUp><<<persistent_grid(), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_shape& s, const bf16_t* h, const int32_t* offsets,
                            const bf16_t* wd, const bf16_t* wsd, bf16_t* y_perm,
                            bf16_t* y_shared, hipStream_t st) {
  GemmArgs a;
  a.a_routed = h;
  a.gather = nullptr;
  a.a_shared = h + static_cast<size_t>(s.T) * s.k * s.F;
  a.w_routed = wd;
  a.w_shared = wsd;
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
  grouped_gemm_kernel<kDown><<<persistent_grid(), kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
