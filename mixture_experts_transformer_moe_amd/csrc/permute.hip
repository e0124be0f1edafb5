// Expert-order permutation: the single-GPU form of the dispatch that the pages
// fuse into their grouped GEMM ("copy expert tokens in expert order", "Laguna
// M.1/XS.2 Technical Report", Key claims, report section 3.1.2, Fig. 2).
//
// Two index kernels and one copy, all deterministic (integer work only; LDS
// atomics count and set bits, which gives the same result in any order):
//   hist    one block per 256 tokens: per-block expert histogram -> workspace
//           (a batch of at most 256 tokens runs both in a single block)
//   scatter one block per 256 tokens: from all the blocks' histograms, each
//           block derives the per-expert totals, their exclusive scan over the
//           experts and its own first position of each expert's tokens (block
//           0 also writes counts and offsets); the rank of token t among the
//           block's tokens of expert e is a popcount over an LDS bitmap of
//           which tokens chose e; position = block base + rank, so each
//           expert's tokens end up in ascending token order
//   gather  x_perm[p] = x[sorted_token[p]] with 16-byte loads and stores,
//           flattened over all (row, chunk) pairs
// A negative expert index marks a slot that is not routed (a padding token):
// it takes no position, its slot_of is -1, and offsets[E] is the number of
// routed slots.
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTB = 256;        // tokens per block
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;       // the router's limit on k
static_assert(kTB == kMaxE, "the scatter kernel keeps one thread per expert");

__device__ __forceinline__ int clamp_e(int e, int E) { return e >= E ? E - 1 : e; }

// Inclusive scan of one value per thread over a block of kTB threads: lane
// shuffles within each wave, then the totals of the waves before (wtot: one
// LDS word per wave).  Ends with every wave total read; the caller
// synchronises before wtot is written again.
__device__ __forceinline__ int block_inclusive_scan(int v, int32_t* wtot) {
  const int ln = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(v, d);
    if (ln >= d) v += n;
  }
  if (ln == 63) wtot[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += wtot[i];
  return v;
}

__global__ __launch_bounds__(kTB) void perm_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int E, int k, int32_t* __restrict__ blk) {
  __shared__ int32_t hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kTB) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kTB + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = clamp_e(idx[static_cast<size_t>(t) * k + j], E);
      if (e >= 0) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kTB) blk[static_cast<size_t>(blockIdx.x) * E + e] = hist[e];
}

// Thread e of every block: expert e's total over all nb blocks and its count
// in the blocks before this one, then an exclusive scan of the totals over
// the experts in LDS.
__global__ __launch_bounds__(kTB) void perm_scatter_kernel(const int32_t* __restrict__ idx, int T,
                                                           int E, int k, int nb,
                                                           const int32_t* __restrict__ blk,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_token,
                                                           int32_t* __restrict__ slot_of) {
  __shared__ uint32_t chose[kMaxE][kTB / 32];   // bit (t mod 256) of row e: token chose e
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t wtot[kTB / 64];
  const int e = threadIdx.x;                      // kTB == kMaxE: one thread per expert
  const int local = threadIdx.x;                  // and one per token of the block
  const int t = blockIdx.x * kTB + local;
  // the token's experts, loaded first so that their latency overlaps the
  // histogram sums and the scan
  int ej[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    ej[j] = (t < T && j < k) ? clamp_e(idx[static_cast<size_t>(t) * k + j], E) : -1;
  for (int i = threadIdx.x; i < kMaxE * (kTB / 32); i += kTB) (&chose[0][0])[i] = 0u;
  int total = 0, before = 0;
  if (e < E) {
    int b = 0;
    for (; b + 8 <= nb; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        total += c[u];
        before += b + u < static_cast<int>(blockIdx.x) ? c[u] : 0;
      }
    }
    for (; b < nb; ++b) {
      const int c = blk[static_cast<size_t>(b) * E + e];
      total += c;
      before += b < static_cast<int>(blockIdx.x) ? c : 0;
    }
  }
  // inclusive scan over the expert totals
  const int incl = block_inclusive_scan(total, wtot);
  const int excl = incl - total;
  base[e] = excl + before;
  if (blockIdx.x == 0 && e < E) {
    counts[e] = total;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = incl;
  }
  __syncthreads();
  const int word = local >> 5;
  const uint32_t bit = 1u << (local & 31);
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (ej[j] >= 0) atomicOr(&chose[ej[j]][word], bit);
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) continue;
      const int ex = ej[j];
      if (ex < 0) {
        slot_of[static_cast<size_t>(t) * k + j] = -1;
        continue;
      }
      int rank = __popc(chose[ex][word] & (bit - 1u));
      for (int w = 0; w < word; ++w) rank += __popc(chose[ex][w]);
      const int pos = base[ex] + rank;
      slot_of[static_cast<size_t>(t) * k + j] = pos;
      sorted_token[pos] = t;
    }
  }
}

// All of it in one block when the batch is one block of tokens (T <= 256,
// decode-sized): the histogram, the scan over the experts and the scatter,
// without the workspace round trip and the second launch.
__global__ __launch_bounds__(kTB) void perm_single_block_kernel(const int32_t* __restrict__ idx, int T,
                                                                int E, int k,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_token,
                                                                int32_t* __restrict__ slot_of) {
  __shared__ uint32_t chose[kMaxE][kTB / 32];   // bit t of row e: token t chose e
  __shared__ int32_t hist[kMaxE];
  __shared__ int32_t scan[kMaxE];
  __shared__ int32_t wtot[kTB / 64];
  const int t = threadIdx.x;                      // token, and expert for the scan
  for (int i = t; i < kMaxE * (kTB / 32); i += kTB) (&chose[0][0])[i] = 0u;
  hist[t] = 0;
  __syncthreads();
  const int word = t >> 5;
  const uint32_t bit = 1u << (t & 31);
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = clamp_e(idx[static_cast<size_t>(t) * k + j], E);
      if (e < 0) continue;
      atomicAdd(&hist[e], 1);
      atomicOr(&chose[e][word], bit);
    }
  __syncthreads();
  const int total = hist[t];
  scan[t] = block_inclusive_scan(total, wtot);
  __syncthreads();
  if (t < E) {
    counts[t] = total;
    offsets[t] = scan[t] - total;
    if (t == E - 1) offsets[E] = scan[t];
  }
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = clamp_e(idx[static_cast<size_t>(t) * k + j], E);
      if (e < 0) {
        slot_of[static_cast<size_t>(t) * k + j] = -1;
        continue;
      }
      int rank = __popc(chose[e][word] & (bit - 1u));
      for (int w = 0; w < word; ++w) rank += __popc(chose[e][w]);
      const int pos = scan[e] - hist[e] + rank;
      slot_of[static_cast<size_t>(t) * k + j] = pos;
      sorted_token[pos] = t;
    }
  }
}

// Copies rows in 16-byte chunks; row_vec = chunks per row.
__global__ __launch_bounds__(256) void perm_gather_kernel(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_token,
                                                          u32x4* __restrict__ x_perm, int64_t total,
                                                          int row_vec, int T) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; c + 3 * stride < total; c += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t cc = c + u * stride;
      const int64_t p = cc / row_vec;
      const int col = static_cast<int>(cc - p * row_vec);
      const int t = min(max(sorted_token[p], 0), T - 1);
      v[u] = x[static_cast<int64_t>(t) * row_vec + col];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x_perm[c + u * stride] = v[u];
  }
  for (; c < total; c += stride) {
    const int64_t p = c / row_vec;
    const int col = static_cast<int>(c - p * row_vec);
    const int t = min(max(sorted_token[p], 0), T - 1);
    x_perm[c] = x[static_cast<int64_t>(t) * row_vec + col];
  }
}

}  // namespace

// Scratch of the entry point that allocates nothing (moe_permute_static): the
// per-block expert histograms in a device array of fixed size.  Each GPU the
// library runs on holds its own copy until the process ends; its address is
// looked up once per device with that device current and kept per device (the
// array's name is a host-side stand-in, never an address to hand a kernel).
// Nothing in it needs clearing: the histogram kernel writes every entry the
// scatter kernel then reads.
constexpr size_t kStaticScratchBytes = size_t{1} << 20;
static __device__ __align__(256) int32_t scratch[kStaticScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

size_t permute_workspace_bytes(const moe_shape& s) {
  const size_t nb = (static_cast<size_t>(s.T) + kTB - 1) / kTB;
  const size_t b = nb * static_cast<size_t>(s.E) * sizeof(int32_t);
  return (b + 255) / 256 * 256;
}

hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* slot_of,
                          void* x_perm, void* workspace, hipStream_t st) {
  const int nb = (s.T + kTB - 1) / kTB;
  int32_t* blk = static_cast<int32_t*>(workspace);
  const int S = s.T * s.k;
  hipError_t err;
  if (nb == 1) {
    perm_single_block_kernel<<<1, kTB, 0, st>>>(idx, s.T, s.E, s.k, counts, offsets,
                                                sorted_token, slot_of);
  } else {
    perm_hist_kernel<<<nb, kTB, 0, st>>>(idx, s.T, s.E, s.k, blk);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    perm_scatter_kernel<<<nb, kTB, 0, st>>>(idx, s.T, s.E, s.k, nb, blk, counts, offsets,
                                            sorted_token, slot_of);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (x_perm) {
    const int elem = s.dtype == MOE_BF16 ? 2 : 4;
    const int row_vec = s.D * elem / 16;
    const int64_t total = static_cast<int64_t>(S) * row_vec;
    const int64_t want = (total + 256 * 4 - 1) / (256 * 4);
    const int blocks = static_cast<int>(want < 16384 ? (want > 0 ? want : 1) : 16384);
    perm_gather_kernel<<<blocks, 256, 0, st>>>(static_cast<const u32x4*>(x), sorted_token,
                                               static_cast<u32x4*>(x_perm), total, row_vec, s.T);
  }
  return hipGetLastError();
}

}  // namespace moe
