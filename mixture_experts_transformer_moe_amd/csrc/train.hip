// Training pass of the MoE layer: the elementwise and per-token kernels around
// the grouped GEMMs.  Readings of the pages ("Laguna M.1/XS.2 Technical
// Report": report summary and Key claims for the router, the 2.5 routed scale
// and the global-batch auxiliary loss; the report thread for padding tokens,
// which are neither routed nor load balanced):
//   * a padding token takes no slot (expert -1, slot -1); its output is the
//     shared expert's alone and its logit gradient is zero;
//   * load statistics over the N routed tokens: f_e = c_e / sum c (counts of
//     the global batch, this batch's by default), p_e = mean over the routed
//     tokens of sigma(z_te) / sum_e' sigma(z_te'); L_aux = beta E sum_e f_e p_e,
//     whose gradient flows through p only;
//   * backward of out_t = y_shared_t + alpha sum_j w_j y_j with the top-k held
//     fixed: dy_j = alpha w_j dout_t, g_j = alpha <dout_t, y_j>, then the
//     renormalisation and the sigmoid: ds_j = (g_j - sum_i w_i g_i) / sum_i s_i,
//     dz_{e_j} = ds_j s_j (1 - s_j); the auxiliary loss adds, for every expert
//     m of a routed token, (c_m - sum_i c_i s'_i) / Q sigma_m (1 - sigma_m) with
//     c = beta E f / N, Q = sum_e sigma_e, s' = sigma / Q.
//
// Every reduction runs in a fixed order (per-thread sums in index order, a
// fixed shuffle tree, waves in order, blocks in order), so results are
// bit-reproducible.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;
constexpr int kDzLd = 256;        // row stride of the bf16 logit gradient (E padded to 256)
constexpr int kStatRows = 16;     // token rows per block of the column sums
constexpr int kMaxE = 256;        // the experts a router row holds at most

__device__ __forceinline__ void load8(const bf16_t* p, float* v) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void store8(bf16_t* p, const float* v) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *reinterpret_cast<u32x4*>(p) = o;
}

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// Sum over the 64 lanes of a wave by a fixed xor tree; every lane gets it.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Rows of the two-part activation buffers: routed rows 0 .. offsets[E] - 1 of
// an [S, w] block, then the T shared rows of a [T, ws] block right after it.
// Item i of a flattened loop is 8 columns of one row.
struct RowItem {
  bool shared;
  int row, col, width;
};

__device__ __forceinline__ bool row_item(int64_t i, int64_t n_routed_items, int w8, int ws8,
                                         int routed_rows, RowItem& it) {
  it.shared = i >= n_routed_items;
  const int64_t j = it.shared ? i - n_routed_items : i;
  const int per = it.shared ? ws8 : w8;
  it.row = static_cast<int>(j / per);
  it.col = 8 * static_cast<int>(j - static_cast<int64_t>(it.row) * per);
  it.width = 8 * per;
  return it.shared || it.row < routed_rows;
}

// h = silu(g) u from the stored pre-activations [g | u]: fp32 math, one rounding.
__global__ __launch_bounds__(256) void swiglu_pre_kernel(const bf16_t* __restrict__ gu,
                                                         bf16_t* __restrict__ h,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         int S, int F, int T, int Fs) {
  const int routed = min(max(offsets[E], 0), S);
  const int64_t nr = static_cast<int64_t>(S) * (F / 8), ns = static_cast<int64_t>(T) * (Fs / 8);
  const bf16_t* gu_s = gu + static_cast<size_t>(S) * 2 * F;
  bf16_t* h_s = h + static_cast<size_t>(S) * F;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nr + ns;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    RowItem it;
    if (!row_item(i, nr, F / 8, Fs / 8, routed, it)) continue;
    const bf16_t* src = (it.shared ? gu_s : gu) + static_cast<size_t>(it.row) * 2 * it.width + it.col;
    float g[8], u[8], o[8];
    load8(src, g);
    load8(src + it.width, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = g[e] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[e])) * u[e];
    store8((it.shared ? h_s : h) + static_cast<size_t>(it.row) * it.width + it.col, o);
  }
}

// SwiGLU backward: dg = dh u silu'(g), du = dh silu(g), silu'(g) = sigma(g) (1 + g (1 - sigma(g))).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16_t* __restrict__ dh,
                                                         const bf16_t* __restrict__ gu,
                                                         bf16_t* __restrict__ dgu,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         int S, int F, int T, int Fs) {
  const int routed = min(max(offsets[E], 0), S);
  const int64_t nr = static_cast<int64_t>(S) * (F / 8), ns = static_cast<int64_t>(T) * (Fs / 8);
  const size_t gu_shared = static_cast<size_t>(S) * 2 * F, dh_shared = static_cast<size_t>(S) * F;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nr + ns;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    RowItem it;
    if (!row_item(i, nr, F / 8, Fs / 8, routed, it)) continue;
    const size_t grow = (it.shared ? gu_shared : 0) + static_cast<size_t>(it.row) * 2 * it.width + it.col;
    const size_t hrow = (it.shared ? dh_shared : 0) + static_cast<size_t>(it.row) * it.width + it.col;
    float g[8], u[8], d[8], dg[8], du[8];
    load8(gu + grow, g);
    load8(gu + grow + it.width, u);
    load8(dh + hrow, d);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[e]));
      dg[e] = d[e] * u[e] * sg * (1.0f + g[e] * (1.0f - sg));
      du[e] = d[e] * g[e] * sg;
    }
    store8(dgu + grow, dg);
    store8(dgu + grow + it.width, du);
  }
}

// Block-wide sum of one value per thread (NW waves): fixed xor tree inside
// each wave, then the wave sums in order.  Every thread gets the result.
template <int NW = 4>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += red[w];
  return r;
}

// Combine backward, one workgroup per token: the output gradients of the
// token's k expert rows (dy_perm, rows in expert order), the routing-weight
// gradients, and the logit gradient row (fp32, and bf16 padded to 256
// columns for the products with the router weights).  A padding token's
// slots are all -1: its logit gradient is zero; a slot < 0 in a routed token
// (not produced by the router) is left out, as if absent.
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ y_perm,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const float* __restrict__ logits,
    const float* __restrict__ coef, bf16_t* __restrict__ dy_perm, float* __restrict__ dz,
    bf16_t* __restrict__ dz16, int D, int k, int E, int S, float alpha) {
  __shared__ int slot_s[kMaxK];
  __shared__ int e_s[kMaxK];
  __shared__ float w_s[kMaxK];
  __shared__ float dot_s[4][kMaxK];
  __shared__ float dsel_s[kMaxK];
  __shared__ float z_s[kDzLd];
  __shared__ int kv_s;
  __shared__ float red4[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < k) {
    slot_s[tid] = min(slot_of[static_cast<size_t>(t) * k + tid], S - 1);
    e_s[tid] = topk_idx[static_cast<size_t>(t) * k + tid];
    w_s[tid] = topk_w[static_cast<size_t>(t) * k + tid];
  }
  // the token's logits, one per thread, loaded together
  const float z = tid < E ? logits[static_cast<size_t>(t) * E + tid] : 0.f;
  z_s[tid] = z;
  __syncthreads();
  if (tid == 0) {
    // keep the routed slots (slot and expert in range), in slot order
    int kv = 0;
    for (int j = 0; j < k; ++j) {
      if (slot_s[j] < 0 || e_s[j] < 0 || e_s[j] >= E) continue;
      slot_s[kv] = slot_s[j];
      e_s[kv] = e_s[j];
      w_s[kv] = w_s[j];
      ++kv;
    }
    kv_s = kv;
  }
  __syncthreads();
  const int kv = kv_s;
  const bool routed = kv > 0;
  if (!routed) {
    for (int e = tid; e < kDzLd; e += 256) {
      if (e < E) dz[static_cast<size_t>(t) * E + e] = 0.f;
      dz16[static_cast<size_t>(t) * kDzLd + e] = 0;
    }
    return;
  }
  // dy rows and the dot products <dout_t, y_j>, 8 columns per thread and step
  float part[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) part[j] = 0.f;
  for (int c = tid * 8; c < D; c += 256 * 8) {
    float d[8];
    load8(dout + static_cast<size_t>(t) * D + c, d);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= kv) continue;
      const size_t row = static_cast<size_t>(slot_s[j]) * D + c;
      float y[8], o[8];
      load8(y_perm + row, y);
      float acc = 0.f;
      const float cj = alpha * w_s[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc = fmaf(d[e], y[e], acc);
        o[e] = cj * d[e];
      }
      part[j] += acc;
      store8(dy_perm + row, o);
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= kv) continue;
    const float v = wave_sum(part[j]);
    if (lane == 0) dot_s[wave][j] = v;
  }
  __syncthreads();
  if (tid == 0) {
    // renormalisation and sigmoid backward over the k slots, in slot order
    float s[kMaxK], g[kMaxK];
    float ssum = 0.f, wg = 0.f;
    for (int j = 0; j < kv; ++j) {
      s[j] = sigmoidf(z_s[e_s[j]]);
      g[j] = alpha * (((dot_s[0][j] + dot_s[1][j]) + dot_s[2][j]) + dot_s[3][j]);
      ssum += s[j];
      wg = fmaf(w_s[j], g[j], wg);
    }
    for (int j = 0; j < kv; ++j) dsel_s[j] = (g[j] - wg) / ssum * s[j] * (1.0f - s[j]);
  }
  __syncthreads();
  // logit gradient row: the auxiliary loss for every expert, plus the slots
  const int e = tid;
  float v = 0.f;
  if (coef != nullptr) {
    const float sg = e < E ? sigmoidf(z) : 0.f;
    const float ce = e < E ? coef[e] : 0.f;
    const float q = block_sum(sg, red4);
    const float cs = block_sum(ce * sg, red4);       // sum_e c_e sigma_e = Q sum_e c_e s'_e
    v = e < E ? (ce - cs / q) / q * sg * (1.0f - sg) : 0.f;
  }
  for (int j = 0; j < kv; ++j)
    if (e_s[j] == e) v += dsel_s[j];
  if (e < E) dz[static_cast<size_t>(t) * E + e] = v;
  dz16[static_cast<size_t>(t) * kDzLd + e] = e < E ? f32_to_bf16(v) : 0;
}

// dx_t = dx_shared_t + dx_router_t + sum over the routed slots of dx_perm rows,
// fp32 in that order, one rounding.
__global__ __launch_bounds__(256) void dx_reduce_kernel(const bf16_t* __restrict__ dx_perm,
                                                        const bf16_t* __restrict__ dx_shared,
                                                        const bf16_t* __restrict__ dx_router,
                                                        const int32_t* __restrict__ slot_of,
                                                        bf16_t* __restrict__ dx, int D, int k, int S) {
  __shared__ int slot_s[kMaxK];
  __shared__ int kv_s;
  const int t = blockIdx.x;
  if (threadIdx.x < k) slot_s[threadIdx.x] = slot_of[static_cast<size_t>(t) * k + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    int kv = 0;
    for (int j = 0; j < k; ++j)
      if (slot_s[j] >= 0) slot_s[kv++] = min(slot_s[j], S - 1);
    kv_s = kv;
  }
  __syncthreads();
  const int kv = kv_s;
  for (int c = threadIdx.x * 8; c < D; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    if (dx_shared) {
      load8(dx_shared + static_cast<size_t>(t) * D + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    load8(dx_router + static_cast<size_t>(t) * D + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
    for (int j = 0; j < kv; ++j) {
      load8(dx_perm + static_cast<size_t>(slot_s[j]) * D + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(dx + static_cast<size_t>(t) * D + c, acc);
  }
}

// Per block of 64 tokens: sum over the block's routed tokens of the
// normalised scores sigma(z_te) / Q_t (stats = true), or of an fp32 [T, E]
// matrix's rows (stats = false), one thread per expert, tokens in order.
template <bool kStats>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const float* __restrict__ m,
                                                             const int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ part, int T, int E,
                                                             int k) {
  __shared__ float q_s[kStatRows];
  const int t0 = blockIdx.x * kStatRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (kStats) {
    // Q_t = sum_e sigma(z_te); 0 marks a padding token (or a row past T).
    // The wave's rows r = wave + 4 i, lane's experts e = lane + 64 j: every
    // load first (all in flight), then the sums in the same order as a plain
    // loop would take them.
    constexpr int kRowsPerWave = kStatRows / 4;
    float z[kRowsPerWave][kMaxE / 64];
    int first[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int t = t0 + wave + 4 * i;
      first[i] = t < T ? topk_idx[static_cast<size_t>(t) * k] : -1;
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j) {
        const int e = lane + 64 * j;
        z[i][j] = (t < T && e < E) ? m[static_cast<size_t>(t) * E + e] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = wave + 4 * i, t = t0 + r;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j)
        if (t < T && lane + 64 * j < E) s += sigmoidf(z[i][j]);
      s = wave_sum(s);
      if (lane == 0) q_s[r] = (t < T && first[i] >= 0) ? s : 0.f;
    }
    __syncthreads();
  }
  const int e = tid;
  if (e >= E) return;
  // the column's rows, all loads in flight, then added in row order
  float v[kStatRows];
#pragma unroll
  for (int r = 0; r < kStatRows; ++r) {
    const int t = t0 + r;
    v[r] = t < T ? m[static_cast<size_t>(t) * E + e] : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < kStatRows; ++r) {
    if (t0 + r >= T) continue;
    if (kStats) {
      if (q_s[r] > 0.f) acc += sigmoidf(v[r]) / q_s[r];
    } else {
      acc += v[r];
    }
  }
  part[static_cast<size_t>(blockIdx.x) * E + e] = acc;
}

// Column sums over the partial rows, 4 threads per expert (1024 threads):
// thread (e, w) adds rows b = w, w + 4, ... in order, 8 loads in flight, and
// the 4 sums are added in w order -- a fixed order, so the result is
// reproducible bit for bit.
constexpr int kFinalThreads = 1024;

__device__ __forceinline__ float colsum4(const float* __restrict__ part, int nb, int E, float* red) {
  const int e = threadIdx.x & 255, w = threadIdx.x >> 8;
  float acc = 0.f;
  if (e < E) {
    int b = w;
    for (; b + 28 < nb; b += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[static_cast<size_t>(b + 4 * u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; b < nb; b += 4) acc += part[static_cast<size_t>(b) * E + e];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  return ((red[e] + red[256 + e]) + red[512 + e]) + red[768 + e];
}

__global__ __launch_bounds__(kFinalThreads) void colsum_final_kernel(const float* __restrict__ part, int nb,
                                                                     int E, float* __restrict__ out) {
  __shared__ float red[kFinalThreads];
  const float v = colsum4(part, nb, E, red);
  if (threadIdx.x < E) out[threadIdx.x] = v;
}

// f, p, the auxiliary loss and its per-expert coefficients c = beta E f / N.
__global__ __launch_bounds__(kFinalThreads) void load_stats_final_kernel(
    const float* __restrict__ part, int nb, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ counts_global, int T, int E, int k, float beta, float* __restrict__ f,
    float* __restrict__ p, float* __restrict__ loss, float* __restrict__ coef) {
  __shared__ float red[kFinalThreads];
  __shared__ float red16[kFinalThreads / 64];
  constexpr int kNW = kFinalThreads / 64;
  const float psum = colsum4(part, nb, E, red);
  // the rest is per expert: threads 0..255, the others adding zeros
  const int e = threadIdx.x;
  // an empty batch has no routed token (its counts buffer was not written)
  const float cl = e < E && T > 0 ? static_cast<float>(counts[e]) : 0.f;
  const float cg = e < E ? (counts_global ? static_cast<float>(counts_global[e]) : cl) : 0.f;
  const float n_slots = block_sum<kNW>(cl, red16);  // counts are exact in fp32 below 2^24
  const float g_slots = block_sum<kNW>(cg, red16);
  const float N = n_slots / static_cast<float>(k);
  const float pe = N > 0.f ? psum / N : 0.f;
  const float fe = g_slots > 0.f ? cg / g_slots : 0.f;
  const float l = block_sum<kNW>(e < E ? fe * pe : 0.f, red16);
  if (e < E) {
    f[e] = fe;
    p[e] = pe;
    coef[e] = N > 0.f ? beta * static_cast<float>(E) * fe / N : 0.f;
  }
  if (e == 0) loss[0] = beta * static_cast<float>(E) * l;
}

int flat_blocks(int64_t items) {
  const int64_t want = (items + 255) / 256;
  return static_cast<int>(want < 8192 ? (want > 0 ? want : 1) : 8192);
}

}  // namespace

size_t train_workspace_bytes(const moe_shape& s) {
  const size_t nb = (static_cast<size_t>(s.T) + kStatRows - 1) / kStatRows;
  const size_t b = nb * static_cast<size_t>(s.E) * sizeof(float);
  return (b + 255) / 256 * 256;
}

hipError_t launch_swiglu_pre(const moe_shape& s, const bf16_t* gu, const int32_t* offsets, bf16_t* h,
                             hipStream_t st) {
  const int64_t items = static_cast<int64_t>(s.T) * s.k * (s.F / 8) + static_cast<int64_t>(s.T) * (s.Fs / 8);
  swiglu_pre_kernel<<<flat_blocks(items), 256, 0, st>>>(gu, h, offsets, s.E, s.T * s.k, s.F, s.T, s.Fs);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const moe_shape& s, const bf16_t* dh, const bf16_t* gu,
                             const int32_t* offsets, bf16_t* dgu, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(s.T) * s.k * (s.F / 8) + static_cast<int64_t>(s.T) * (s.Fs / 8);
  swiglu_bwd_kernel<<<flat_blocks(items), 256, 0, st>>>(dh, gu, dgu, offsets, s.E, s.T * s.k, s.F, s.T, s.Fs);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_shape& s, const bf16_t* dout, const bf16_t* y_perm,
                              const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w,
                              const float* logits, const float* coef, bf16_t* dy_perm, float* dz,
                              bf16_t* dz16, hipStream_t st) {
  combine_bwd_kernel<<<s.T, 256, 0, st>>>(dout, y_perm, slot_of, topk_idx, topk_w, logits, coef, dy_perm,
                                          dz, dz16, s.D, s.k, s.E, s.T * s.k, s.alpha);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const moe_shape& s, const bf16_t* dx_perm, const bf16_t* dx_shared,
                            const bf16_t* dx_router, const int32_t* slot_of, bf16_t* dx, hipStream_t st) {
  dx_reduce_kernel<<<s.T, 256, 0, st>>>(dx_perm, dx_shared, dx_router, slot_of, dx, s.D, s.k, s.T * s.k);
  return hipGetLastError();
}

hipError_t launch_load_stats(const moe_shape& s, const float* logits, const int32_t* topk_idx,
                             const int32_t* counts, const int32_t* counts_global, float beta, float* f,
                             float* p, float* loss, float* coef, void* ws, hipStream_t st) {
  const int nb = (s.T + kStatRows - 1) / kStatRows;
  float* part = static_cast<float*>(ws);
  if (nb > 0) {
    colsum_partial_kernel<true><<<nb, 256, 0, st>>>(logits, topk_idx, part, s.T, s.E, s.k);
    if (hipError_t e = hipGetLastError()) return e;
  }
  load_stats_final_kernel<<<1, kFinalThreads, 0, st>>>(part, nb, counts, counts_global, s.T, s.E, s.k, beta, f,
                                                      p, loss, coef);
  return hipGetLastError();
}

hipError_t launch_colsum(const moe_shape& s, const float* m, float* out, void* ws, hipStream_t st) {
  const int nb = (s.T + kStatRows - 1) / kStatRows;
  float* part = static_cast<float*>(ws);
  if (nb > 0) {
    colsum_partial_kernel<false><<<nb, 256, 0, st>>>(m, nullptr, part, s.T, s.E, s.k);
    if (hipError_t e = hipGetLastError()) return e;
  }
  colsum_final_kernel<<<1, kFinalThreads, 0, st>>>(part, nb, s.E, out);
  return hipGetLastError();
}

}  // namespace moe
