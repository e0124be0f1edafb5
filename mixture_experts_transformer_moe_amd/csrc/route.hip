// Router of the MoE layer: logits, token-choice top-k and renormalised sigmoid
// weights ("Laguna M.1/XS.2 Technical Report", Key claims: sigmoid router,
// token-choice top-8 of 256, post-top-k normalization; report section 3.1).
//
// Two kernels.
//   logits  bf16: blocks of tokens x experts on MFMA, fp32 accumulation, the
//           bias added once, fp32 logits stored (route_bf16_kernel below).
//           fp32: one wave per token, plain fp32 FMA in index order.
//   top-k   one 16-lane DPP row per token (4 tokens per wave); lane c holds
//           the candidates e = c + 16 i.  Each of the k rounds takes the
//           largest key among the candidates not yet taken (row maximum over
//           an order-preserving uint32 image of z), then the lowest index
//           holding it (row minimum), and zeroes that candidate's key, so the
//           order is (z descending, index ascending) exactly and independent
//           of timing.  Sigmoid of the selected logits, renormalised over the
//           k slots.
#include <type_traits>

#include "lds_dma.h"

namespace moe {
namespace {


// Monotone map of fp32 onto uint32 (larger z -> larger key); -0.0 is folded
// onto +0.0 first so that the two zeros tie.
__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The value a key came from (-0.0 comes back as +0.0).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Row-wide (16 lanes) reduction of an associative, commutative operation
// through DPP row rotations: after rotating by 1, 2, 4 and 8 lanes every lane
// of the row holds the result.
template <typename Op>
__device__ __forceinline__ uint32_t row_allreduce_u32(uint32_t v, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x121, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x122, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xf, 0xf, false)));
  return v;
}

// Row sum: lane 15 of each row after DPP row shifts, read back by readlane and
// handed to every lane of the row (one summation order for the whole row).
__device__ __forceinline__ float row_sum_f32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
  const int b0 = __builtin_amdgcn_readlane(__float_as_int(v), 15), b1 = __builtin_amdgcn_readlane(__float_as_int(v), 31);
  const int b2 = __builtin_amdgcn_readlane(__float_as_int(v), 47), b3 = __builtin_amdgcn_readlane(__float_as_int(v), 63);
  const int row = (threadIdx.x & 63) >> 4;
  return __int_as_float(row == 0 ? b0 : row == 1 ? b1 : row == 2 ? b2 : b3);
}

constexpr int kXcds = 8;                       // workgroup b runs on XCD b mod 8
constexpr int kTopkThreads = 256;              // 4 waves x 4 tokens
constexpr int kTopkTokens = kTopkThreads / 16;

// Top-k of the stored logits, 16 lanes per token (E <= 256, k <= 16).  A
// token whose mask byte is 0 (padding) is not routed: expert -1, weight 0.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits,
                                                            const uint8_t* __restrict__ mask,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ wout, int T, int E, int k) {
  const int c = threadIdx.x & 15;
  const int t_raw = blockIdx.x * kTopkTokens + (threadIdx.x >> 4);
  const int t = min(t_raw, T - 1);                 // rows past T compute a copy of the last one
  const float* z = logits + static_cast<size_t>(t) * E;
  // keys of the candidates still in the running; 0 marks one taken or absent
  // (real keys are >= 1)
  uint32_t key[16];
  // all 16 loads unconditional (clamped index), so that they are in flight
  // together
  float zv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) zv[i] = z[min(c + 16 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < 16; ++i) key[i] = order_key(zv[i]) & (c + 16 * i < E ? ~0u : 0u);
  int my_e = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, key[i]);
    const uint32_t best = row_allreduce_u32(m, [](uint32_t a, uint32_t b) { return max(a, b); });
    // the lowest index holding the best key
    uint32_t cand = 0xffffu;
#pragma unroll
    for (int i = 15; i >= 0; --i)
      if (key[i] == best) cand = static_cast<uint32_t>(c + 16 * i);
    const int e = static_cast<int>(row_allreduce_u32(cand, [](uint32_t a, uint32_t b) { return min(a, b); }));
    // taken: key zeroed in the lane that holds it
    const int taken_i = (e & 15) == c ? e >> 4 : 16;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (taken_i == i) key[i] = 0u;
    if (c == j) {
      my_e = e;
      my_key = best;
    }
  }
  // sigmoid of the selected logits (the exact fp32 values, recovered from
  // their keys), renormalised
  const float s = c < k ? 1.0f / (1.0f + expf(-key_value(my_key))) : 0.f;
  const float sum = row_sum_f32(s);
  const bool routed = mask == nullptr || mask[t] != 0;
  if (t_raw < T && c < k) {
    idx[static_cast<size_t>(t) * k + c] = routed ? my_e : -1;
    wout[static_cast<size_t>(t) * k + c] = routed ? s / sum : 0.f;
  }
}

// Router logits, bf16: a workgroup of NW waves (4, or 8 for the large blocks)
// computes a TM x TN block of logits (tokens x experts) over the whole of D.
// Wave w sits at (tm, tn, ks):
// it owns WM x WN MF x MF blocks (tokens WM tm .., experts WN tn ..; WM = WN =
// 2 in the largest block shape, so each fragment read from LDS feeds two
// MFMAs) and, when the four waves split K (KS = 4 for small batches, so that
// few tokens still keep 4 load streams per CU), the K blocks ks, ks + KS, ...;
// the partial blocks are summed in LDS in ks order.  Token rows and router rows reach LDS by direct global->LDS loads
// (each covers 8 rows x 128 bytes, XOR-swizzled) through a ring of NS stages
// of KS 64-wide K blocks, the same number of loads per wave in every stage, so
// every wait is a constant.  MFMA with the router rows as the first operand:
// 32 x 32 blocks (v_mfma_f32_32x32x16_bf16): lane l holds token (l mod 32),
// register quads 4 adjacent experts; 16 x 16 blocks (TM = TN = 16, for the
// smallest batches: 4 times the workgroups, each reading half the rows;
// v_mfma_f32_16x16x32_bf16): lane l holds token (l mod 16) and experts
// 4 (l / 16) + 0..3.
template <int TM, int TN, int KS, int NS, int NW = 4, int WM = 1, int WN = 1>
__global__ __launch_bounds__(64 * NW, 1) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T, int D,
                                                            int E) {
  constexpr int MF = TM < 32 ? 16 : 32;                // MFMA block edge
  constexpr int kRows = TM + TN;                       // rows per K block: tokens, then experts
  constexpr int kBlockElems = kRows * kPipeBK;
  constexpr int kStageElems = KS * kBlockElems;
  constexpr int kLoads = KS * kRows / 8;               // 1 KB loads per stage
  constexpr int LPW = kLoads / NW;                     // per wave
  static_assert((TM / (MF * WM)) * (TN / (MF * WN)) * KS == NW && kLoads % NW == 0,
                "NW waves, equal loads per stage");
  static_assert(MF == 32 || (TM == 16 && TN == 16), "16 x 16 blocks: one per wave");
  static_assert(KS == 1 || WM * WN == 1, "split K: one block per wave");
  static_assert(NS * kStageElems * 2 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) bf16_t lds[NS * kStageElems];
  const int tiles_n = (E + TN - 1) / TN;
  // blocks numbered token block-major and dealt to the XCDs in runs of
  // consecutive numbers (XCD x takes the x-th run, one block per workgroup it
  // runs), so that the blocks of one token block share an L2 and read its
  // token rows from HBM once (dealt round-robin they were read once per
  // expert block)
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcds;
  const int tile = xcd * (G / kXcds) + min(xcd, G % kXcds) + blockIdx.x / kXcds;
  const int t0 = (tile / tiles_n) * TM;
  const int e0 = (tile % tiles_n) * TN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ks = wave % KS;
  const int tm = (wave / KS) % (TM / (MF * WM));
  const int tn = (wave / KS) / (TM / (MF * WM));
  const int NKB = D / kPipeBK;                         // a multiple of KS

  // this lane's LPW loads per stage: load q of wave w is load i = LPW w + q of
  // the stage: K block i / (kRows / 8), rows 8 (i mod (kRows / 8)) + 0..7 of it
  const bf16_t* src[LPW];
  uint32_t dst_off[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int i = LPW * wave + q;
    const int kb = i / (kRows / 8);
    const int P = (i % (kRows / 8)) * 64 + lane;       // chunk slot inside the K block
    int row, col;
    chunk_source(P, row, col);
    const bf16_t* r = row < TM ? x + static_cast<size_t>(min(t0 + row, T - 1)) * D
                               : wr + static_cast<size_t>(min(e0 + row - TM, E - 1)) * D;
    src[q] = r + kb * kPipeBK + col;
    dst_off[q] = static_cast<uint32_t>((kb * kBlockElems + (i % (kRows / 8)) * 512) * 2);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  // stage s holds K blocks s KS .. s KS + KS - 1
  const int nst = NKB / KS;
  // workgroups that share router rows start at different K offsets, so that
  // they do not all ask the same L2 lines for the same block at once (each
  // token's sum is still taken in one fixed order)
  const int rot = (tile / tiles_n) % nst;
  auto issue = [&](int slot, int s) {
    const uint32_t base = lds0 + static_cast<uint32_t>(slot * kStageElems * 2);
    const int sr = s + rot < nst ? s + rot : s + rot - nst;
#pragma unroll
    for (int q = 0; q < LPW; ++q)
      dma16(src[q] + static_cast<size_t>(sr) * KS * kPipeBK, __builtin_amdgcn_readfirstlane(base + dst_off[q]));
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s, min(s, nst - 1));

  using Acc = std::conditional_t<MF == 32, f32x16, f32x4>;
  constexpr int NR = MF == 32 ? 16 : 4;                // accumulator registers
  Acc acc[WM][WN];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int n = 0; n < WN; ++n) acc[m][n] = Acc{0.f};
  int arow[WM], brow[WN];
#pragma unroll
  for (int m = 0; m < WM; ++m) arow[m] = MF * (WM * tm + m) + (lane & (MF - 1));
#pragma unroll
  for (int n = 0; n < WN; ++n) brow[n] = TM + MF * (WN * tn + n) + (lane & (MF - 1));
  int slot = 0;
  for (int s = 0; s < nst; ++s) {
    // this stage was issued NS - 1 stages ago; the NS - 2 later ones (LPW
    // loads each) may still be in flight
    __builtin_amdgcn_s_waitcnt(vmcnt_only(LPW * (NS - 2)));
    __builtin_amdgcn_s_barrier();
    issue(slot == 0 ? NS - 1 : slot - 1, min(s + NS - 1, nst - 1));
    const bf16_t* blk = lds + slot * kStageElems + ks * kBlockElems;
    // all fragments of the block first: one LDS latency per block, not per
    // step.  A step covers 16 (32 x 32 blocks) or 32 (16 x 16) of the 64 K
    // values; lane l takes 16-byte chunk l / MF of the step's chunks.
    constexpr int kSteps = MF == 32 ? 4 : 2;
    bf16x8 fa[WM][kSteps], fb[WN][kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int ch = (8 / kSteps) * i + lane / MF;
#pragma unroll
      for (int n = 0; n < WN; ++n)
        fb[n][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&blk[pipe_swz(brow[n], ch)]));
#pragma unroll
      for (int m = 0; m < WM; ++m)
        fa[m][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&blk[pipe_swz(arow[m], ch)]));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSteps; ++i)
#pragma unroll
      for (int m = 0; m < WM; ++m)
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          if constexpr (MF == 32)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[n][i], fa[m][i], acc[m][n], 0, 0, 0);
          else
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[n][i], fa[m][i], acc[m][n], 0, 0, 0);
        }
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  // the tail loads (clamped repeats) land before LDS is reused or the
  // workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  if constexpr (KS > 1) {
    __builtin_amdgcn_s_barrier();
    float* red = reinterpret_cast<float*>(lds);        // [KS][NR][64]
#pragma unroll
    for (int r = 0; r < NR; ++r) red[(ks * NR + r) * 64 + lane] = acc[0][0][r];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float v = red[r * 64 + lane];
#pragma unroll
      for (int j = 1; j < KS; ++j) v += red[(j * NR + r) * 64 + lane];
      acc[0][0][r] = v;
    }
  }
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    const int t = t0 + MF * (WM * tm + m) + (lane & (MF - 1));
    if (t >= T) continue;
#pragma unroll
    for (int n = 0; n < WN; ++n)
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        // 4 adjacent experts
        const int e = e0 + MF * (WN * tn + n) + (MF == 32 ? mfma32_row(4 * q, lane) : 4 * (lane >> 4));
        float z[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          z[c] = acc[m][n][4 * q + c] + ((bias && e + c < E) ? bias[min(e + c, E - 1)] : 0.f);
        float* dst = logits + static_cast<size_t>(t) * E + e;
        if ((E & 3) == 0 && e + 4 <= E) {
          *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
        } else {
          for (int c = 0; c < 4; ++c)
            if (e + c < E) dst[c] = z[c];
        }
      }
  }
}

// fp32 path: one wave per token, logits by plain fp32 FMA in index order.
__global__ __launch_bounds__(64) void route_f32_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ wr,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits, int T, int D, int E) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* xr = x + static_cast<size_t>(t) * D;
  for (int e = lane; e < E; e += 64) {
    const float* w = wr + static_cast<size_t>(e) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(xr[d], w[d], acc);
    logits[static_cast<size_t>(t) * E + e] = acc + (bias ? bias[e] : 0.f);
  }
}

}  // namespace

hipError_t launch_topk(const moe_shape& s, const float* logits, const uint8_t* mask, int32_t* idx,
                       float* w, hipStream_t st) {
  const int blocks = (s.T + kTopkTokens - 1) / kTopkTokens;
  topk_kernel<<<blocks, kTopkThreads, 0, st>>>(logits, mask, idx, w, s.T, s.E, s.k);
  return hipGetLastError();
}

hipError_t launch_route_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wr,
                             const float* bias, const uint8_t* mask, float* logits, int32_t* idx,
                             float* w, hipStream_t st) {
  // 128 x 64 blocks of 8 waves when there are at least as many as CUs, else
  // 64 x 64 blocks when they are enough to fill the chip, else 32 x 32 blocks
  // with the K split over the workgroup's waves, else (fewer than half as many
  // as there are CUs) 16 x 16 blocks.  The stages are few: the
  // loads in flight per CU do not grow past a few stages' worth, and every
  // stage beyond that adds clamped repeat loads at the end of the K loop
  // (measured: 4 stages 11 to 16% faster than 8 on 8192 and 32768 tokens)
  const int huge = ((s.T + 127) / 128) * ((s.E + 63) / 64);
  const int big = ((s.T + 63) / 64) * ((s.E + 63) / 64);
  const int mid = ((s.T + 31) / 32) * ((s.E + 31) / 32);
  if (s.E == 256 && (s.T + 127) / 128 >= 256) {
    // all 256 experts of 128 tokens per workgroup, each wave 64 x 64 (every
    // fragment read from LDS feeds two MFMAs): half the bytes into LDS per
    // logit of the 128 x 64 blocks, and still a block per CU
    route_bf16_kernel<128, 256, 1, 3, 8, 2, 2><<<(s.T + 127) / 128, 512, 0, st>>>(x, wr, bias, logits, s.T,
                                                                                s.D, s.E);
  } else if (huge >= 256) {
    // 128 x 64 blocks, 8 waves: a quarter fewer bytes into LDS per logit
    route_bf16_kernel<128, 64, 1, 4, 8><<<huge, 512, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  } else if (big >= 128) {
    route_bf16_kernel<64, 64, 1, 4><<<big, 256, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  } else if (mid >= 128) {
    route_bf16_kernel<32, 32, 4, 4><<<mid, 256, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  } else {
    const int blocks = ((s.T + 15) / 16) * ((s.E + 15) / 16);
    route_bf16_kernel<16, 16, 4, 4><<<blocks, 256, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  }
  if (hipError_t e = hipGetLastError()) return e;
  return launch_topk(s, logits, mask, idx, w, st);
}

hipError_t launch_route_f32(const moe_shape& s, const float* x, const float* wr,
                            const float* bias, const uint8_t* mask, float* logits, int32_t* idx,
                            float* w, hipStream_t st) {
  route_f32_kernel<<<s.T, 64, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_topk(s, logits, mask, idx, w, st);
}

}  // namespace moe
