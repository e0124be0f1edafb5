// Router of the MoE layer: logits, token-choice top-k and renormalised sigmoid
// weights ("Laguna M.1/XS.2 Technical Report", Key claims: sigmoid router,
// token-choice top-8 of 256, post-top-k normalization; report section 3.1).
//
// bf16 path: one workgroup of 4 waves per 32 tokens.  Wave w owns experts
// [64w, 64w+64) and accumulates the 32 x 64 logit block with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation) in the shared pipelined loop
// (mma_pipeline.h): token rows and router-weight rows (hot in L2) stream into
// LDS through a ring of direct global->LDS loads.  The bias is added once,
// the fp32 logits are stored, and the same values are staged in LDS for the
// selection.
//
// Selection: one wave per token, k rounds of a DPP wave maximum over an
// order-preserving uint32 image of the logits, ties resolved to the lower
// expert index by ballots; exact and independent of timing.
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

// Maximum of v over the wave: DPP shifts inside each row of 16 lanes, then the
// four row maxima through readlane.  The result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  return max(max(r0, r1), max(r2, r3));
}

// One wave selects the top-k of zrow[0..E) and writes slot order + weights.
// Lane l holds candidates e = l + 64 i (i < 4).  Each round takes the largest
// key among the candidates not yet taken (wave max), then the lowest index
// holding it (ballots scanned in index order), so the order is (z descending,
// index ascending) exactly, whatever the values (non-finite ones included).
__device__ void wave_topk(const float* zrow, int E, int k, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[4];
  uint32_t taken = 0;                       // bit i: candidate i taken or absent
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(zrow[e]) : 0u;
    if (e >= E) taken |= 1u << i;
  }
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!((taken >> i) & 1u)) m = max(m, key[i]);
    const uint32_t best = wave_max_u32(m);
    int e = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned long long b = __ballot(!((taken >> i) & 1u) && key[i] == best);
      if (!found && b != 0ull) {
        e = 64 * i + __ffsll(b) - 1;
        found = true;
      }
    }
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
    if (lane == j) my_e = e;
  }
  float s = 0.f;
  if (lane < k) s = 1.0f / (1.0f + expf(-zrow[my_e]));
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __shfl(s, j, 64);    // slot order
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = s / sum;
  }
}

template <int NS>
__global__ __launch_bounds__(256, 1) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ wout, int T, int D,
                                                            int E, int k) {
  using PT = PipeTile<kRouteTokens, kMaxE>;
  constexpr int kLdsElems = NS * PT::kStageElems;
  static_assert(kRouteTokens * (kMaxE + 1) * 2 <= kLdsElems, "logit tile fits the ring");
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
  float (*zs)[kMaxE + 1] = reinterpret_cast<float (*)[kMaxE + 1]>(lds);
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
          zs[row][e0 + c] = z[c];
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
  __syncthreads();
  for (int r = wave; r < kRouteTokens; r += 4) {
    const int t = t0 + r;
    if (t < T) wave_topk(zs[r], E, k, idx + static_cast<size_t>(t) * k, wout + static_cast<size_t>(t) * k);
  }
}

// fp32 path: one wave per token, logits by plain fp32 FMA in index order.
__global__ __launch_bounds__(64) void route_f32_kernel(const float* __restrict__ x,
                                                       const float* __restrict__ wr,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ wout, int T, int D,
                                                       int E, int k) {
  __shared__ float zs[kMaxE];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* xr = x + static_cast<size_t>(t) * D;
  for (int e = lane; e < E; e += 64) {
    const float* w = wr + static_cast<size_t>(e) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(xr[d], w[d], acc);
    const float z = acc + (bias ? bias[e] : 0.f);
    zs[e] = z;
    logits[static_cast<size_t>(t) * E + e] = z;
  }
  __syncthreads();
  wave_topk(zs, E, k, idx + static_cast<size_t>(t) * k, wout + static_cast<size_t>(t) * k);
}

}  // namespace

hipError_t launch_route_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wr,
                             const float* bias, float* logits, int32_t* idx, float* w,
                             hipStream_t st) {
  const int blocks = (s.T + kRouteTokens - 1) / kRouteTokens;
  route_bf16_kernel<4><<<blocks, 256, 0, st>>>(x, wr, bias, logits, idx, w, s.T, s.D, s.E, s.k);
  return hipGetLastError();
}

hipError_t launch_route_f32(const moe_shape& s, const float* x, const float* wr,
                            const float* bias, float* logits, int32_t* idx, float* w,
                            hipStream_t st) {
  route_f32_kernel<<<s.T, 64, 0, st>>>(x, wr, bias, logits, idx, w, s.T, s.D, s.E, s.k);
  return hipGetLastError();
}

}  // namespace moe
