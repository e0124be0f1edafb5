// Router of the MoE layer: logits, token-choice top-k and renormalised sigmoid
// weights ("Laguna M.1/XS.2 Technical Report", Key claims: sigmoid router,
// token-choice top-8 of 256, post-top-k normalization; report section 3.1).
//
// bf16 path: one workgroup of 4 waves per 32 tokens.  Wave w owns experts
// [64w, 64w+64) and accumulates the 32 x 64 logit block with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation), reading its operand fragments
// straight from global memory (the router weight, E x D, stays hot in L2).  The
// bias is added once, the fp32 logits are stored, and the same values are
// staged in LDS for the selection.
//
// Selection: one wave per token.  Each lane holds up to four candidates
// (e = lane + 64 i) as 64-bit keys that order (z descending, e ascending), with
// -0.0 folded onto +0.0.  k rounds of a wave-wide max pick the slots in order,
// so the result is exact and does not depend on timing.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteTokens = 32;
constexpr int kMaxE = 256;

__device__ __forceinline__ uint64_t order_key(float z, int e) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;                          // -0.0 == +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);        // monotone in z
  // low half: larger for lower expert index; always >= 0xFF00, so a valid key
  // is never 0 (0 marks "taken / absent").
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(0xFFFFu - e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// One wave selects the top-k of zrow[0..E) and writes slot order + weights.
__device__ void wave_topk(const float* zrow, int E, int k, int32_t* idx_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(zrow[e], e) : 0ull;
  }
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = 0xFFFF - static_cast<int>(best & 0xFFFFull);
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i == (e >> 6)) key[i] = 0ull;
    }
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

__global__ __launch_bounds__(256) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ wout, int T, int D,
                                                         int E, int k) {
  __shared__ float zs[kRouteTokens][kMaxE + 1];
  const int t0 = blockIdx.x * kRouteTokens;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int e_base = 64 * wave;

  if (e_base < E) {
    f32x16 acc0 = {0.f}, acc1 = {0.f};
    const int koff = (lane >> 5) * 8;
    const int arow = min(t0 + (lane & 31), T - 1);
    const int brow0 = min(e_base + (lane & 31), E - 1);
    const int brow1 = min(e_base + 32 + (lane & 31), E - 1);
    const bf16_t* pa = x + static_cast<size_t>(arow) * D + koff;
    const bf16_t* pb0 = wr + static_cast<size_t>(brow0) * D + koff;
    const bf16_t* pb1 = wr + static_cast<size_t>(brow1) * D + koff;
    for (int k0 = 0; k0 < D; k0 += 16) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(pa + k0);
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(pb0 + k0);
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(pb1 + k0);
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b0), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8, b1), acc1, 0, 0, 0);
    }
    // C layout of the 32x32 MFMA: lane holds column (lane & 31), register i holds
    // row (i / 4) * 8 + (lane / 32) * 4 + (i % 4).
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = e_base + 32 * nb + (lane & 31);
      if (col < E) {
        const float b = bias ? bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          const float z = (nb == 0 ? acc0[i] : acc1[i]) + b;
          zs[r][col] = z;
          if (t0 + r < T) logits[static_cast<size_t>(t0 + r) * E + col] = z;
        }
      }
    }
  }
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
  route_bf16_kernel<<<blocks, 256, 0, st>>>(x, wr, bias, logits, idx, w, s.T, s.D, s.E, s.k);
  return hipGetLastError();
}

hipError_t launch_route_f32(const moe_shape& s, const float* x, const float* wr,
                            const float* bias, float* logits, int32_t* idx, float* w,
                            hipStream_t st) {
  route_f32_kernel<<<s.T, 64, 0, st>>>(x, wr, bias, logits, idx, w, s.T, s.D, s.E, s.k);
  return hipGetLastError();
}

}  // namespace moe
