// Combine: out[t] = y_shared[t] + sum_j (alpha * w[t,j]) * y_perm[slot_of[t,j]]
// ("Laguna M.1/XS.2 Technical Report", Key claims: routed-expert output
// modulated by 2.5 before combining with the shared expert).  A weighted gather
// of k expert-ordered rows per token, fp32 accumulation in slot order, one
// rounding.  HBM-bound: one workgroup per token, 16-byte loads; the shared add
// is fused.  The y_perm rows are read exactly once, so they are loaded
// non-temporally: cached normally they push the output rows out of L2 and MALL
// before those are written back (measured at 32768 tokens x 2048: 5.1 TB/s
// with cached loads, 6.1 TB/s with non-temporal ones).  Slots with slot_of < 0 (a padding token, not routed) are skipped,
// so such a token's output is the shared expert's alone.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

__global__ __launch_bounds__(256) void combine_bf16_kernel(const bf16_t* __restrict__ y_perm,
                                                           const bf16_t* __restrict__ y_shared,
                                                           const int32_t* __restrict__ slot_of,
                                                           const float* __restrict__ topk_w,
                                                           bf16_t* __restrict__ out, int D, int k,
                                                           int S, float alpha) {
  __shared__ int slot_s[kMaxK];
  __shared__ float coef_s[kMaxK];
  __shared__ int kv_s;
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    slot_s[threadIdx.x] = slot_of[static_cast<size_t>(t) * k + threadIdx.x];
    coef_s[threadIdx.x] = alpha * topk_w[static_cast<size_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // keep the routed slots, in slot order
    int kv = 0;
    for (int j = 0; j < k; ++j) {
      const int p = slot_s[j];
      if (p < 0) continue;
      slot_s[kv] = min(p, S - 1);
      coef_s[kv] = coef_s[j];
      ++kv;
    }
    kv_s = kv;
  }
  __syncthreads();
  const int kv = __builtin_amdgcn_readfirstlane(kv_s);
  for (int c = threadIdx.x * 8; c < D; c += blockDim.x * 8) {
    // the shared row's chunk first: it needs no routing
    u32x4 sh = {0u, 0u, 0u, 0u};
    if (y_shared) sh = *reinterpret_cast<const u32x4*>(y_shared + static_cast<size_t>(t) * D + c);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // the routed rows in batches of 8: a batch's loads all in flight together
    // (a small batch of tokens has too few workgroups to hide one load's
    // latency per slot), then the products in slot order
    for (int j0 = 0; j0 < kv; j0 += 8) {
      u32x4 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        q[u] = j0 + u < kv ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                 y_perm + static_cast<size_t>(slot_s[j0 + u]) * D + c))
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= kv) continue;
        const float cj = coef_s[j0 + u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(cj, __uint_as_float(q[u][i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(cj, __uint_as_float(q[u][i] & 0xffff0000u), acc[2 * i + 1]);
        }
      }
    }
    if (y_shared) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __uint_as_float(sh[i] << 16) + acc[2 * i];
        acc[2 * i + 1] = __uint_as_float(sh[i] & 0xffff0000u) + acc[2 * i + 1];
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4*>(out + static_cast<size_t>(t) * D + c) = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y_perm,
                                                          const float* __restrict__ y_shared,
                                                          const int32_t* __restrict__ slot_of,
                                                          const float* __restrict__ topk_w,
                                                          float* __restrict__ out, int D, int k,
                                                          int S, float alpha) {
  __shared__ int slot_s[kMaxK];
  __shared__ float coef_s[kMaxK];
  __shared__ int kv_s;
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    slot_s[threadIdx.x] = slot_of[static_cast<size_t>(t) * k + threadIdx.x];
    coef_s[threadIdx.x] = alpha * topk_w[static_cast<size_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // keep the routed slots, in slot order
    int kv = 0;
    for (int j = 0; j < k; ++j) {
      const int p = slot_s[j];
      if (p < 0) continue;
      slot_s[kv] = min(p, S - 1);
      coef_s[kv] = coef_s[j];
      ++kv;
    }
    kv_s = kv;
  }
  __syncthreads();
  const int kv = kv_s;
  for (int c = threadIdx.x * 4; c < D; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < kv; ++j) {
      const f32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(y_perm + static_cast<size_t>(slot_s[j]) * D + c));
      const float cj = coef_s[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(cj, v[i], acc[i]);
    }
    if (y_shared) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(y_shared + static_cast<size_t>(t) * D + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = v[i] + acc[i];
    }
    *reinterpret_cast<f32x4*>(out + static_cast<size_t>(t) * D + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                          const int32_t* slot_of, const float* topk_w, void* out,
                          hipStream_t st) {
  if (s.dtype == MOE_BF16)
    combine_bf16_kernel<<<s.T, 256, 0, st>>>(static_cast<const bf16_t*>(y_perm),
                                             static_cast<const bf16_t*>(y_shared), slot_of, topk_w,
                                             static_cast<bf16_t*>(out), s.D, s.k, s.T * s.k, s.alpha);
  else
    combine_f32_kernel<<<s.T, 256, 0, st>>>(static_cast<const float*>(y_perm),
                                            static_cast<const float*>(y_shared), slot_of, topk_w,
                                            static_cast<float*>(out), s.D, s.k, s.T * s.k, s.alpha);
  return hipGetLastError();
}

}  // namespace moe
