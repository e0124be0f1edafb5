// fp32 expert FFN (small fp32 layers, held to 1e-5 relative): one workgroup per
// expert-ordered row, the row staged in LDS, each thread one output column with
// fp32 FMA in index order.  Same contract as the bf16 grouped GEMMs, weights in
// the same packed layout ("Laguna-M.1-base", Feed-forward: SwiGLU, no biases).
#include "moe_internal.h"   // packed_offset

namespace moe {
namespace {

constexpr int kMaxRow = 8192;   // floats staged per row (validated on the host)

__device__ __forceinline__ int expert_of(const int32_t* offsets, int E, int p) {
  int lo = 0, hi = E - 1;       // last e with offsets[e] <= p
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(const float* __restrict__ a_routed,
                                                          const int32_t* __restrict__ gather,
                                                          const float* __restrict__ x,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ wgu,
                                                          const float* __restrict__ wsgu,
                                                          float* __restrict__ h, int S, int T,
                                                          int E, int D, int F, int Fs) {
  __shared__ float arow[kMaxRow];
  const int p = blockIdx.x;
  const bool shared = p >= S;
  const float* src;
  const float* w;
  int n;
  float* out;
  if (!shared) {
    const int e = expert_of(offsets, E, p);
    src = gather ? x + static_cast<size_t>(min(max(gather[p], 0), T - 1)) * D
                 : a_routed + static_cast<size_t>(p) * D;
    w = wgu + static_cast<size_t>(e) * packed_matrix_elems(2 * F, D);
    n = F;
    out = h + static_cast<size_t>(p) * F;
  } else {
    const int t = p - S;
    src = x + static_cast<size_t>(t) * D;
    w = wsgu;
    n = Fs;
    out = h + static_cast<size_t>(S) * F + static_cast<size_t>(t) * Fs;
  }
  for (int d = threadIdx.x; d < D; d += blockDim.x) arow[d] = src[d];
  __syncthreads();
  for (int f = threadIdx.x; f < n; f += blockDim.x) {
    float gv = 0.f, uv = 0.f;
    for (int d = 0; d < D; ++d) {
      gv = fmaf(w[packed_offset(f, d, D)], arow[d], gv);
      uv = fmaf(w[packed_offset(n + f, d, D)], arow[d], uv);
    }
    out[f] = gv / (1.0f + expf(-gv)) * uv;
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ h,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ wd,
                                                       const float* __restrict__ wsd,
                                                       float* __restrict__ y_perm,
                                                       float* __restrict__ y_shared, int S, int E,
                                                       int D, int F, int Fs) {
  __shared__ float hrow[kMaxRow];
  const int p = blockIdx.x;
  const bool shared = p >= S;
  const float* src;
  const float* w;
  int kdim;
  float* out;
  if (!shared) {
    const int e = expert_of(offsets, E, p);
    src = h + static_cast<size_t>(p) * F;
    w = wd + static_cast<size_t>(e) * packed_matrix_elems(D, F);
    kdim = F;
    out = y_perm + static_cast<size_t>(p) * D;
  } else {
    const int t = p - S;
    src = h + static_cast<size_t>(S) * F + static_cast<size_t>(t) * Fs;
    w = wsd;
    kdim = Fs;
    out = y_shared + static_cast<size_t>(t) * D;
  }
  for (int f = threadIdx.x; f < kdim; f += blockDim.x) hrow[f] = src[f];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int f = 0; f < kdim; ++f) acc = fmaf(w[packed_offset(d, f, kdim)], hrow[f], acc);
    out[d] = acc;
  }
}

}  // namespace

hipError_t launch_gate_up_f32(const moe_shape& s, const float* x_perm,
                              const int32_t* sorted_token, const float* x,
                              const int32_t* offsets, const float* wgu, const float* wsgu,
                              float* h, hipStream_t st) {
  const int S = s.T * s.k;
  const int rows = S + (s.Fs > 0 ? s.T : 0);
  gate_up_f32_kernel<<<rows, 256, 0, st>>>(x_perm ? x_perm : x, x_perm ? nullptr : sorted_token,
                                           x, offsets, wgu, wsgu, h, S, s.T, s.E, s.D, s.F, s.Fs);
  return hipGetLastError();
}

hipError_t launch_down_f32(const moe_shape& s, const float* h, const int32_t* offsets,
                           const float* wd, const float* wsd, float* y_perm, float* y_shared,
                           hipStream_t st) {
  const int S = s.T * s.k;
  const int rows = S + (s.Fs > 0 ? s.T : 0);
  down_f32_kernel<<<rows, 256, 0, st>>>(h, offsets, wd, wsd, y_perm, y_shared, S, s.E, s.D, s.F,
                                        s.Fs);
  return hipGetLastError();
}

}  // namespace moe
