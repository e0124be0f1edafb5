// Weight gradients of the MoE layer: for each group g and its token rows R_g,
//   dW[m][n] = sum_{r in R_g} A[r][m] B[r][n]
// with, per group (the chain rule of "Laguna-M.1-base", Feed-forward: SwiGLU
// without biases, and of the router of "Laguna M.1/XS.2 Technical Report",
// Key claims):
//   routed expert e, gate/up   A = [dg | du] rows of e,  B = x rows of e's tokens  -> dW_gu[e] [2F, D]
//   routed expert e, down      A = dy rows of e,         B = h rows of e           -> dW_d[e]  [D, F]
//   shared expert, gate/up     A = [dg | du]_shared,     B = x (all T rows)        -> dW_sgu   [2Fs, D]
//   shared expert, down        A = dout,                 B = h_shared              -> dW_sd    [D, Fs]
//   router                     A = dz (bf16, 256 wide),  B = x                     -> dW_r     [E, D] fp32
// bf16 operands, fp32 accumulation; expert gradients rounded once to bf16,
// the router's kept in fp32.  A group with no rows gets zeros.
//
// Design.  The reduction runs over token rows, which are the strided
// dimension of both operands, while a 32x32x16 MFMA wants 8 consecutive K
// values per lane.  Each stage therefore moves 64 token rows of a 128-column
// A tile and a 128-column B tile through LDS transposed: a thread loads 16
// bytes (8 columns) from each of 4 consecutive rows, pairs the rows' values
// column by column with v_perm, and writes 8-byte [column][4 rows] pieces
// (ds_write_b64, 16 lanes = one contiguous 128-byte run); the fragments then
// come back as single 16-byte LDS reads.  LDS rows are 72 elements (144 bytes)
// long, so the 8 lanes of a 16-byte read hit 8 disjoint bank groups.  A tile
// is 128 x 128 outputs, 4 waves of 64 x 64 (2 x 2 MFMA blocks); the MFMA's
// first operand is the B fragment, so a lane holds consecutive output columns
// and stores 16 bytes after a lane-pair swap, as in the forward GEMMs.  Two
// LDS stages (72 KB) let the next stage's loads fly during the MFMAs.
//
// Schedule: the long groups (shared expert, router: all T rows) and the
// routed experts' tiles are dealt to the 8 XCDs so that each XCD gets an
// equal share of the long tiles first, then the tiles of a contiguous run of
// experts (blocks b and b + 8 run on the same XCD), so an expert's rows are
// read into one L2.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTile = 128;            // output tile edge (M and N)
constexpr int kKC = 64;               // token rows per stage
constexpr int kRowE = 72;             // LDS row length in elements (64 rows + 8 pad)
constexpr int kOpElems = kTile * kRowE;
constexpr int kStageElems = 2 * kOpElems;   // A then B
constexpr int kXcds = 8;
constexpr int kDzLd = 256;

struct WgradArgs {
  const bf16_t* x;             // [T, D]
  const int32_t* gather;       // sorted_token: row p of a routed expert is token gather[p] ...
  const bf16_t* x_perm;        // ... or, when not null, row p of x_perm [S, D]
  const bf16_t* dgu;           // [S, 2F] routed, then [T, 2Fs] shared
  const bf16_t* dy;            // [S, D]
  const bf16_t* h;             // [S, F] routed, then [T, Fs] shared
  const bf16_t* dout;          // [T, D]
  const bf16_t* dz16;          // [T, 256]
  const int32_t* offsets;      // [E + 1]
  bf16_t* dwgu;                // [E, 2F, D]
  bf16_t* dwd;                 // [E, D, F]
  bf16_t* dwsgu;               // [2Fs, D]
  bf16_t* dwsd;                // [D, Fs]
  float* dwr;                  // [E, D]
  int T, D, E, F, Fs, S;
  int n_router, n_sgu, n_sd;   // long tiles of each long group
  int long_per_xcd;
  int tiles_gu, tiles_d;       // tiles of one routed expert's two matrices
  int experts_per_xcd;
};

struct TileJob {
  const bf16_t* a;             // A element (row r, column m0 + c) at a + r * lda + c
  const bf16_t* b;             // B element at b + row(r) * ldb + c
  int lda, ldb;
  bool gathered;               // B rows through gather[]
  int r0, r1;                  // token rows
  void* out;                   // output element (m0 + i, n0 + j) at out + i * ldo + j
  int ldo;
  int m_valid;                 // rows of the tile inside the matrix
  bool f32;
};

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile: block b runs on XCD b % 8 as the (b / 8)-th of its blocks
  const int xcd = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
  TileJob j{};
  int m0, n0;
  if (i < g.long_per_xcd) {
    const int li = xcd + kXcds * i;
    if (li >= g.n_router + g.n_sgu + g.n_sd) return;
    j.r0 = 0;
    j.r1 = g.T;
    j.gathered = false;
    if (li < g.n_router) {
      const int nt = g.D / kTile;
      m0 = (li / nt) * kTile;
      n0 = (li % nt) * kTile;
      j.a = g.dz16 + m0;
      j.lda = kDzLd;
      j.b = g.x + n0;
      j.ldb = g.D;
      j.out = g.dwr + static_cast<size_t>(m0) * g.D + n0;
      j.ldo = g.D;
      j.m_valid = min(kTile, g.E - m0);
      j.f32 = true;
    } else if (li < g.n_router + g.n_sgu) {
      const int t = li - g.n_router, nt = g.D / kTile;
      m0 = (t / nt) * kTile;
      n0 = (t % nt) * kTile;
      j.a = g.dgu + static_cast<size_t>(g.S) * 2 * g.F + m0;
      j.lda = 2 * g.Fs;
      j.b = g.x + n0;
      j.ldb = g.D;
      j.out = g.dwsgu + static_cast<size_t>(m0) * g.D + n0;
      j.ldo = g.D;
      j.m_valid = kTile;
      j.f32 = false;
    } else {
      const int t = li - g.n_router - g.n_sgu, nt = g.Fs / kTile;
      m0 = (t / nt) * kTile;
      n0 = (t % nt) * kTile;
      j.a = g.dout + m0;
      j.lda = g.D;
      j.b = g.h + static_cast<size_t>(g.S) * g.F + n0;
      j.ldb = g.Fs;
      j.out = g.dwsd + static_cast<size_t>(m0) * g.Fs + n0;
      j.ldo = g.Fs;
      j.m_valid = kTile;
      j.f32 = false;
    }
  } else {
    const int ri = i - g.long_per_xcd;
    const int tpe = g.tiles_gu + g.tiles_d;
    const int e = xcd * g.experts_per_xcd + ri / tpe;
    if (ri / tpe >= g.experts_per_xcd || e >= g.E) return;
    const int t = ri % tpe;
    j.r0 = g.T > 0 ? min(max(g.offsets[e], 0), g.S) : 0;
    j.r1 = g.T > 0 ? min(max(g.offsets[e + 1], j.r0), g.S) : 0;
    j.m_valid = kTile;
    j.f32 = false;
    if (t < g.tiles_gu) {
      const int nt = g.D / kTile;
      m0 = (t / nt) * kTile;
      n0 = (t % nt) * kTile;
      j.a = g.dgu + m0;
      j.lda = 2 * g.F;
      j.gathered = g.x_perm == nullptr;
      j.b = (j.gathered ? g.x : g.x_perm) + n0;
      j.ldb = g.D;
      j.out = g.dwgu + (static_cast<size_t>(e) * 2 * g.F + m0) * g.D + n0;
      j.ldo = g.D;
    } else {
      const int u = t - g.tiles_gu, nt = g.F / kTile;
      m0 = (u / nt) * kTile;
      n0 = (u % nt) * kTile;
      j.a = g.dy + m0;
      j.lda = g.D;
      j.gathered = false;
      j.b = g.h + n0;
      j.ldb = g.F;
      j.out = g.dwd + (static_cast<size_t>(e) * g.D + m0) * g.F + n0;
      j.ldo = g.F;
    }
  }
  (void)m0;
  (void)n0;

  // ---- stage loads: thread (kq, seg) takes rows 4 kq .. 4 kq + 3 of the
  // stage and columns 8 seg .. 8 seg + 7 of both operands
  const int kq = tid & 15, seg = tid >> 4;
  u32x4 ra[4], rb[4];
  auto load_stage = [&](int r_first) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r_first + 4 * kq + q;
      const bool in = r < j.r1;
      const int rr = in ? r : j.r0;          // any row of the group: not used
      int brow = rr;
      if (j.gathered) brow = min(max(g.gather[rr], 0), g.T - 1);
      const u32x4 va = *reinterpret_cast<const u32x4*>(j.a + static_cast<size_t>(rr) * j.lda + 8 * seg);
      const u32x4 vb = *reinterpret_cast<const u32x4*>(j.b + static_cast<size_t>(brow) * j.ldb + 8 * seg);
      ra[q] = in ? va : u32x4{0u, 0u, 0u, 0u};
      rb[q] = in ? vb : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // transposed write: column c = 8 seg + 2 d + h of the tile, rows 4 kq .. 4 kq + 3
  auto store_stage = [&](bf16_t* st) {
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const u32x4* v = op == 0 ? ra : rb;
      bf16_t* base = st + op * kOpElems + 4 * kq;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint2 lo = make_uint2(lo_pair(v[0][d], v[1][d]), lo_pair(v[2][d], v[3][d]));
        const uint2 hi = make_uint2(hi_pair(v[0][d], v[1][d]), hi_pair(v[2][d], v[3][d]));
        *reinterpret_cast<uint2*>(base + (8 * seg + 2 * d) * kRowE) = lo;
        *reinterpret_cast<uint2*>(base + (8 * seg + 2 * d + 1) * kRowE) = hi;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{0.f};

  const int wm = 64 * (wave & 1), wn = 64 * (wave >> 1);
  const int nch = (j.r1 - j.r0 + kKC - 1) / kKC;
  if (nch > 0) {
    load_stage(j.r0);
    store_stage(lds);
    __syncthreads();
  }
  for (int c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    if (more) load_stage(j.r0 + (c + 1) * kKC);
    const bf16_t* st = lds + (c & 1) * kStageElems;
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = 16 * ks + 8 * (lane >> 5);
        fa[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               st + (wm + 32 * q + (lane & 31)) * kRowE + col));
        fb[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               st + kOpElems + (wn + 32 * q + (lane & 31)) * kRowE + col));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[b], fa[a], acc[a][b], 0, 0, 0);
    }
    if (more) store_stage(lds + ((c + 1) & 1) * kStageElems);
    __syncthreads();
  }

  // ---- epilogue: lane l holds output row wm + 32 a + (l % 32) and, in register
  // quad q of block b, columns wn + 32 b + 8 q + 4 (l / 32) + 0..3
  const int mrow = wm + (lane & 31);
  if (j.f32) {
    float* out = static_cast<float*>(j.out);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int m = mrow + 32 * a;
      if (m >= j.m_valid) continue;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(out + static_cast<size_t>(m) * j.ldo + wn + 32 * b + 8 * q + 4 * (lane >> 5)) =
              make_float4(acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
    }
    return;
  }
  bf16_t* out = static_cast<bf16_t*>(j.out);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int m = mrow + 32 * a;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t v[2][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q = 2 * p + hh;
          v[hh][0] = pack_bf16x2(acc[a][b][4 * q], acc[a][b][4 * q + 1]);
          v[hh][1] = pack_bf16x2(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
        }
        // lanes < 32 keep quad 2p and take the upper lanes' quad 2p; lanes
        // >= 32 take the lower lanes' quad 2p + 1 and keep theirs
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const auto sw = __builtin_amdgcn_permlane32_swap(v[0][cc], v[1][cc], false, false);
          v[0][cc] = sw[0];
          v[1][cc] = sw[1];
        }
        if (m < j.m_valid)
          *reinterpret_cast<uint4*>(out + static_cast<size_t>(m) * j.ldo + wn + 32 * b + 16 * p + 8 * (lane >> 5)) =
              make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
      }
  }
}

}  // namespace

hipError_t launch_wgrad(const moe_shape& s, const bf16_t* x, const int32_t* sorted_token,
                        const bf16_t* x_perm, const bf16_t* dgu, const bf16_t* dy, const bf16_t* h,
                        const bf16_t* dout, const bf16_t* dz16, const int32_t* offsets, bf16_t* dwgu,
                        bf16_t* dwd, bf16_t* dwsgu, bf16_t* dwsd, float* dwr, hipStream_t st) {
  WgradArgs a{};
  a.x = x;
  a.gather = sorted_token;
  a.x_perm = x_perm;
  a.dgu = dgu;
  a.dy = dy;
  a.h = h;
  a.dout = dout;
  a.dz16 = dz16;
  a.offsets = offsets;
  a.dwgu = dwgu;
  a.dwd = dwd;
  a.dwsgu = dwsgu;
  a.dwsd = dwsd;
  a.dwr = dwr;
  a.T = s.T;
  a.D = s.D;
  a.E = s.E;
  a.F = s.F;
  a.Fs = s.Fs;
  a.S = s.T * s.k;
  a.n_router = dwr ? (s.E + kTile - 1) / kTile * (s.D / kTile) : 0;
  a.n_sgu = s.Fs > 0 ? (2 * s.Fs / kTile) * (s.D / kTile) : 0;
  a.n_sd = s.Fs > 0 ? (s.D / kTile) * (s.Fs / kTile) : 0;
  const int n_long = a.n_router + a.n_sgu + a.n_sd;
  a.long_per_xcd = (n_long + kXcds - 1) / kXcds;
  a.tiles_gu = (2 * s.F / kTile) * (s.D / kTile);
  a.tiles_d = (s.D / kTile) * (s.F / kTile);
  a.experts_per_xcd = (s.E + kXcds - 1) / kXcds;
  const int per_xcd = a.long_per_xcd + a.experts_per_xcd * (a.tiles_gu + a.tiles_d);
  wgrad_kernel<<<kXcds * per_xcd, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
