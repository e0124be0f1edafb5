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
// Design.  The reduction runs over token rows, the strided dimension of both
// operands, while a 32x32x16 MFMA wants 8 consecutive K values per lane.
// Stages of 32 token rows of a 256-column A tile and a 128-column B tile go
// from global memory straight into LDS (global_load_lds_dwordx4, no
// registers), row-major, the 16-byte units of row r XOR-swizzled by
// 4 (r mod 4); gfx950's transposing LDS read (ds_read_b64_tr_b16) then hands
// each lane 4 consecutive rows of one column, two reads per MFMA fragment.  In
// a group of 16 lanes that read returns to lane 4a + b element b of the 8-byte
// pieces addressed by lanes a, a + 4, a + 8 and a + 12, so lane j addresses
// row k0 + j / 4, columns c0 + 4 (j mod 4) .. + 3, and lane i receives rows
// k0 .. k0 + 3 of column c0 + i; with the swizzle the 16 lanes of a read hit
// distinct banks.  Three stages are in flight (72 KB, 2 workgroups per CU):
// the tiles are short (an expert's ~100-200 rows are a few stages), so
// several stages must fly at once to cover the load latency.  Rows past the
// group's end load its last row again and the A values of the last stage's
// rows past the end are zeroed, so they add nothing.
// A tile is 256 x 128 outputs, 8 waves of 64 x 64 (2 x 2 MFMA blocks); the
// MFMA's first operand is the B fragment, so a lane holds consecutive output
// columns, 8 of them after a lane-pair swap.  The bf16 tile then goes through
// LDS and out as whole 256-byte rows with non-temporal stores (the router's
// fp32 rows go out directly).  The gradients written (1.6 GB at the XS.2
// shape) dominate the traffic, with the operand rows the tiles re-read.
// Gathered token ids (x rows of a routed expert) come through scalar loads,
// 4 per wave and stage, so that no vector wait drains the stages in flight.
//
// Schedule: the long groups (shared expert, router: all T rows) and the
// routed experts' tiles are dealt to the 8 XCDs so that each XCD gets an
// equal share of the long tiles first, then the tiles of a contiguous run of
// experts (blocks b and b + 8 run on the same XCD), so an expert's rows are
// read into one L2.
#include "lds_dma.h"

namespace moe {
namespace {

constexpr int kBM = 256;              // output tile rows (A columns)
constexpr int kBN = 128;              // output tile columns (B columns)
constexpr int kKC = 32;               // token rows per stage
constexpr int kNS = 3;                // stages in flight
constexpr int kAElems = kKC * kBM;
constexpr int kBElems = kKC * kBN;
constexpr int kStageElems = kAElems + kBElems;
constexpr int kThreadsW = 512;
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

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int unit_swz(int r) { return 4 * (r & 3); }

// element offset of (row, col) in a stage operand of `units` 16-byte units per row
template <int kUnits>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * (8 * kUnits) + (((col >> 3) ^ unit_swz(row)) << 3) + (col & 7);
}

// MFMA fragment of columns c0 .. c0 + 31, rows k0 .. k0 + 15 (lane l: column
// c0 + l mod 32, rows k0 + 8 (l / 32) + 0..7)
template <int kUnits>
__device__ __forceinline__ bf16x8 tr_fragment(const bf16_t* t, int c0, int k0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const int col = c0 + 16 * (grp & 1) + 4 * (j & 3);
  const int row = k0 + 8 * (grp >> 1) + (j >> 2);
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4*)(reinterpret_cast<__attribute__((address_space(3))) bf16_t*>(
          static_cast<uint32_t>(reinterpret_cast<uintptr_t>(t + tile_off<kUnits>(row, col))))));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4*)(reinterpret_cast<__attribute__((address_space(3))) bf16_t*>(
          static_cast<uint32_t>(reinterpret_cast<uintptr_t>(t + tile_off<kUnits>(row + 4, col))))));
  const v4i16 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kThreadsW, 2) void wgrad_kernel(WgradArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[kNS * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile: block b runs on XCD b % 8 as the (b / 8)-th of its blocks
  const int xcd = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
  TileJob j{};
  if (i < g.long_per_xcd) {
    const int li = xcd + kXcds * i;
    if (li >= g.n_router + g.n_sgu + g.n_sd) return;
    j.r0 = 0;
    j.r1 = g.T;
    j.gathered = false;
    int m0, n0;
    if (li < g.n_router) {
      const int nt = g.D / kBN;
      m0 = (li / nt) * kBM;
      n0 = (li % nt) * kBN;
      j.a = g.dz16 + m0;
      j.lda = kDzLd;
      j.b = g.x + n0;
      j.ldb = g.D;
      j.out = g.dwr + static_cast<size_t>(m0) * g.D + n0;
      j.ldo = g.D;
      j.m_valid = min(kBM, g.E - m0);
      j.f32 = true;
    } else if (li < g.n_router + g.n_sgu) {
      const int t = li - g.n_router, nt = g.D / kBN;
      m0 = (t / nt) * kBM;
      n0 = (t % nt) * kBN;
      j.a = g.dgu + static_cast<size_t>(g.S) * 2 * g.F + m0;
      j.lda = 2 * g.Fs;
      j.b = g.x + n0;
      j.ldb = g.D;
      j.out = g.dwsgu + static_cast<size_t>(m0) * g.D + n0;
      j.ldo = g.D;
      j.m_valid = kBM;
      j.f32 = false;
    } else {
      const int t = li - g.n_router - g.n_sgu, nt = g.Fs / kBN;
      m0 = (t / nt) * kBM;
      n0 = (t % nt) * kBN;
      j.a = g.dout + m0;
      j.lda = g.D;
      j.b = g.h + static_cast<size_t>(g.S) * g.F + n0;
      j.ldb = g.Fs;
      j.out = g.dwsd + static_cast<size_t>(m0) * g.Fs + n0;
      j.ldo = g.Fs;
      j.m_valid = kBM;
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
    j.m_valid = kBM;
    j.f32 = false;
    if (t < g.tiles_gu) {
      const int nt = g.D / kBN;
      const int m0 = (t / nt) * kBM, n0 = (t % nt) * kBN;
      j.a = g.dgu + m0;
      j.lda = 2 * g.F;
      j.gathered = g.x_perm == nullptr;
      j.b = (j.gathered ? g.x : g.x_perm) + n0;
      j.ldb = g.D;
      j.out = g.dwgu + (static_cast<size_t>(e) * 2 * g.F + m0) * g.D + n0;
      j.ldo = g.D;
    } else {
      const int u = t - g.tiles_gu, nt = g.F / kBN;
      const int m0 = (u / nt) * kBM, n0 = (u % nt) * kBN;
      j.a = g.dy + m0;
      j.lda = g.D;
      j.gathered = false;
      j.b = g.h + n0;
      j.ldb = g.F;
      j.out = g.dwd + (static_cast<size_t>(e) * g.D + m0) * g.F + n0;
      j.ldo = g.F;
    }
  }

  // ---- stage loads: wave w issues A loads 2w and 2w + 1 (1 KB each = two
  // 512-byte A rows) and B load w (four 256-byte B rows) of every stage
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const int nch = (j.r1 - j.r0 + kKC - 1) / kKC;
  auto issue = [&](int c) {
    const int slot = c % kNS;
    const uint32_t base = lds0 + static_cast<uint32_t>(slot * kStageElems * 2);
    const int rbase = j.r0 + c * kKC;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int P = 64 * (2 * wave + q) + lane;          // A slot: row P / 32, unit slot P % 32
      const int r = P >> 5;
      const int u = (P & 31) ^ unit_swz(r);
      const int row = min(rbase + r, j.r1 - 1);
      dma16(j.a + static_cast<size_t>(row) * j.lda + 8 * u,
            __builtin_amdgcn_readfirstlane(base + static_cast<uint32_t>((2 * wave + q) * 1024)));
    }
    {
      const int P = 64 * wave + lane;                    // B slot: row P / 16, unit slot P % 16
      const int r = P >> 4;
      const int u = (P & 15) ^ unit_swz(r);
      int row = min(rbase + r, j.r1 - 1);
      if (j.gathered) {
        // the wave's 4 rows: token ids by scalar loads
        const __attribute__((address_space(4))) int32_t* gt =
            (const __attribute__((address_space(4))) int32_t*)(g.gather);
        const int rw = rbase + 4 * wave;
        int id[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) id[k] = gt[min(rw + k, j.r1 - 1)];
        int tok = id[0];
#pragma unroll
        for (int k = 1; k < 4; ++k) tok = (lane >> 4) == k ? id[k] : tok;
        row = min(max(tok, 0), g.T - 1);
      }
      dma16(j.b + static_cast<size_t>(row) * j.ldb + 8 * u,
            __builtin_amdgcn_readfirstlane(base + static_cast<uint32_t>(kAElems * 2 + wave * 1024)));
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{0.f};

  const int wm = 64 * (wave & 3), wn = 64 * (wave >> 2);
#pragma unroll
  for (int c = 0; c < kNS - 1; ++c)
    if (c < nch) issue(c);
  for (int c = 0; c < nch; ++c) {
    // stage c landed: the stages issued after it (3 loads each per wave) may fly
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_only(3));
    else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + kNS - 1 < nch) issue(c + kNS - 1);
    const bf16_t* A = lds + (c % kNS) * kStageElems;
    const bf16_t* B = A + kAElems;
    const int kvalid = j.r1 - (j.r0 + c * kKC);          // rows of this stage inside the group
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        fa[q] = tr_fragment<kBM / 8>(A, wm + 32 * q, 16 * ks, lane);
        fb[q] = tr_fragment<kBN / 8>(B, wn + 32 * q, 16 * ks, lane);
      }
      if (kvalid < kKC) {
        // rows past the group's end: zero A (B holds finite repeats)
        const int k0 = 16 * ks + 8 * (lane >> 5);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + e >= kvalid) fa[q][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[b], fa[a], acc[a][b], 0, 0, 0);
    }
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
  // bf16: the tile goes through LDS (rows of 128 outputs, 16-byte units XOR-
  // swizzled by row), then out in whole 256-byte rows, 4 rows per wave
  // store: far fewer cache lines per store than 16-byte pieces of 32 rows
  bf16_t* out = static_cast<bf16_t*>(j.out);
  __syncthreads();                      // every wave is done with the stages
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
        const int u = (wn + 32 * b + 16 * p + 8 * (lane >> 5)) >> 3;
        *reinterpret_cast<uint4*>(lds + m * kBN + ((u ^ (m & 15)) << 3)) =
            make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
      }
  }
  __syncthreads();
  constexpr int kUnitsOut = kBM * kBN / 8;
#pragma unroll
  for (int i = 0; i < kUnitsOut / kThreadsW; ++i) {
    const int idx = tid + kThreadsW * i;
    const int r = idx / (kBN / 8), u = idx % (kBN / 8);
    // non-temporal: the gradients are not read again here, and kept out of
    // L2 they leave it to the operand rows the other tiles re-read
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kBN + ((u ^ (r & 15)) << 3));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * j.ldo + 8 * u));
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
  a.n_router = dwr ? (s.E + kBM - 1) / kBM * (s.D / kBN) : 0;
  a.n_sgu = s.Fs > 0 ? (2 * s.Fs / kBM) * (s.D / kBN) : 0;
  a.n_sd = s.Fs > 0 ? (s.D / kBM) * (s.Fs / kBN) : 0;
  const int n_long = a.n_router + a.n_sgu + a.n_sd;
  a.long_per_xcd = (n_long + kXcds - 1) / kXcds;
  a.tiles_gu = (2 * s.F / kBM) * (s.D / kBN);
  a.tiles_d = (s.D / kBM) * (s.F / kBN);
  a.experts_per_xcd = (s.E + kXcds - 1) / kXcds;
  const int per_xcd = a.long_per_xcd + a.experts_per_xcd * (a.tiles_gu + a.tiles_d);
  wgrad_kernel<<<kXcds * per_xcd, kThreadsW, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
