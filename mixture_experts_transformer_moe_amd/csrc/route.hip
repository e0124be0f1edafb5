// Router of the MoE layer: logits, token-choice top-k and renormalised sigmoid
// weights ("Laguna M.1/XS.2 Technical Report", Key claims: sigmoid router,
// token-choice top-8 of 256, post-top-k normalization; report section 3.1).
//
// Two kernels.
//   logits  bf16: one workgroup of 4 waves per 32 tokens; wave w owns experts
//           [64w, 64w+64) and accumulates the 32 x 64 logit block with
//           v_mfma_f32_32x32x16_bf16 (fp32 accumulation) in the shared
//           pipelined loop (mma_pipeline.h): token rows and router-weight
//           rows (hot in L2) stream into LDS through a ring of direct
//           global->LDS loads.  The bias is added once and the fp32 logits
//           stored.  fp32: one wave per token, plain fp32 FMA in index order.
//   top-k   one 16-lane DPP row per token (4 tokens per wave); lane c holds
//           the candidates e = c + 16 i.  Each of the k rounds takes the
//           largest key among the candidates not yet taken (row maximum over
//           an order-preserving uint32 image of z), then the lowest index
//           holding it (row minimum), so the order is (z descending, index
//           ascending) exactly and independent of timing.  Sigmoid of the
//           selected logits, renormalised over the k slots.
#include "mma_pipeline.h"

namespace moe {
namespace {

constexpr int kRouteTokens = 32;
constexpr int kMaxE = 256;

// Monotone map of fp32 onto uint32 (larger z -> larger key); -0.0 is folded
// onto +0.0 first so that the two zeros tie.
__device__ __forceinline__ uint32_t order_key(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Row-wide (16 lanes) reductions through DPP row shifts: after them lane 15
// of each row holds the row's result, read back by readlane and handed to
// every lane of the row.  `id` is the identity of the operation.
template <typename Op>
__device__ __forceinline__ uint32_t row_reduce_u32(uint32_t v, uint32_t id, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  const int row = (threadIdx.x & 63) >> 4;
  return row == 0 ? r0 : row == 1 ? r1 : row == 2 ? r2 : r3;
}

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

constexpr int kTopkThreads = 256;              // 4 waves x 4 tokens
constexpr int kTopkTokens = kTopkThreads / 16;

// Top-k of the stored logits, 16 lanes per token (E <= 256, k <= 16).
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ wout, int T, int E, int k) {
  const int c = threadIdx.x & 15;
  const int t_raw = blockIdx.x * kTopkTokens + (threadIdx.x >> 4);
  const int t = min(t_raw, T - 1);                 // rows past T compute a copy of the last one
  const float* z = logits + static_cast<size_t>(t) * E;
  uint32_t key[16];
  uint32_t taken = 0;                              // bit i: candidate c + 16 i taken or absent
  // all 16 loads unconditional (clamped index), so that they are in flight
  // together
  float zv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) zv[i] = z[min(c + 16 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = c + 16 * i;
    key[i] = e < E ? order_key(zv[i]) : 0u;        // real keys are >= 1
    if (e >= E) taken |= 1u << i;
  }
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!((taken >> i) & 1u)) m = max(m, key[i]);
    const uint32_t best = row_reduce_u32(m, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
    uint32_t cand = 0xffffu;
#pragma unroll
    for (int i = 15; i >= 0; --i)
      if (!((taken >> i) & 1u) && key[i] == best) cand = static_cast<uint32_t>(c + 16 * i);
    const int e = static_cast<int>(row_reduce_u32(cand, 0xffffu, [](uint32_t a, uint32_t b) { return min(a, b); }));
    if ((e & 15) == c) taken |= 1u << (e >> 4);
    if (c == j) my_e = e;
  }
  // sigmoid of the selected logits (exact fp32 values), renormalised
  const float s = c < k ? 1.0f / (1.0f + expf(-z[my_e])) : 0.f;
  const float sum = row_sum_f32(s);
  if (t_raw < T && c < k) {
    idx[static_cast<size_t>(t) * k + c] = my_e;
    wout[static_cast<size_t>(t) * k + c] = s / sum;
  }
}

template <int NS>
__global__ __launch_bounds__(256, 1) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T, int D,
                                                            int E) {
  using PT = PipeTile<kRouteTokens, kMaxE>;
  constexpr int kLdsElems = NS * PT::kStageElems;
  __shared__ __attribute__((aligned(16))) bf16_t lds[kLdsElems];
  const int t0 = blockIdx.x * kRouteTokens;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int e_base = 64 * wave;
  const int valid = min(kRouteTokens, T - t0);

  const bf16_t* a_src[PT::kAGroups];
  const bf16_t* b_src[PT::kBInst];
  pipe_sources<kRouteTokens, kMaxE>(
      a_src, b_src, [&](int r) { return x + static_cast<size_t>(min(t0 + r, T - 1)) * D; },
      [&](int r) { return wr + static_cast<size_t>(min(r, E - 1)) * D; });
  const int brow[2] = {e_base, e_base + 32};
  mma_pipeline<kRouteTokens, kMaxE, NS>(a_src, b_src, D / kPipeBK, valid, brow, lds, [&](auto& acc) {
    // lane: token (lane & 31); register quad q: experts e0 + 8 q + 4 (lane / 32) + 0..3
    const int row = lane & 31;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e0 = e_base + 32 * j + 8 * q + 4 * (lane >> 5);
        float z[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          z[c] = acc[0][j][4 * q + c] + ((bias && e0 + c < E) ? bias[e0 + c] : 0.f);
        }
        if (row < valid && e0 < E) {
          float* dst = logits + static_cast<size_t>(t0 + row) * E + e0;
          if (e0 + 4 <= E && (E & 3) == 0) {
            *reinterpret_cast<float4*>(dst) = make_float4(z[0], z[1], z[2], z[3]);
          } else {
            for (int c = 0; c < 4 && e0 + c < E; ++c) dst[c] = z[c];
          }
        }
      }
    }
  });
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

hipError_t launch_topk(const moe_shape& s, const float* logits, int32_t* idx, float* w, hipStream_t st) {
  const int blocks = (s.T + kTopkTokens - 1) / kTopkTokens;
  topk_kernel<<<blocks, kTopkThreads, 0, st>>>(logits, idx, w, s.T, s.E, s.k);
  return hipGetLastError();
}

hipError_t launch_route_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wr,
                             const float* bias, float* logits, int32_t* idx, float* w,
                             hipStream_t st) {
  const int blocks = (s.T + kRouteTokens - 1) / kRouteTokens;
  route_bf16_kernel<4><<<blocks, 256, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_topk(s, logits, idx, w, st);
}

hipError_t launch_route_f32(const moe_shape& s, const float* x, const float* wr,
                            const float* bias, float* logits, int32_t* idx, float* w,
                            hipStream_t st) {
  route_f32_kernel<<<s.T, 64, 0, st>>>(x, wr, bias, logits, s.T, s.D, s.E);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_topk(s, logits, idx, w, st);
}

}  // namespace moe
