// Arguments and launch helpers shared by the two grouped-GEMM kernels: the
// weight-streaming kernel (grouped_gemm.hip) and the LDS-tiled kernel for
// batches with many rows per expert (grouped_gemm_lds.hip).
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kGemmMaxE = 256;
constexpr int kGemmXcds = 8;        // workgroup b runs on XCD b mod 8

enum GemmMode { kGateUp = 0, kDown = 1 };

struct GemmArgs {
  const bf16_t* a_routed;   // [S, K] rows in expert order (x_perm or h), or x when gather != null
  const int32_t* gather;    // sorted_token (A row p = x[gather[p]]) or null
  const bf16_t* a_shared;   // [T, Ks]
  const unsigned char* w_routed;   // E packed [Nw, K] matrices (bf16, or FP8 codes)
  const unsigned char* w_shared;   // packed [Nws, Ks]
  const float* s_routed;    // FP8 weights: per-row scales [E, Nw] (else unused)
  const float* s_shared;    //   [Nws]
  bf16_t* out_routed;       // [S, N]
  bf16_t* out_shared;       // [T, Ns]
  const int32_t* offsets;   // [E + 1]
  int T, E, S;
  int K, Ks;                // reduction length (routed / shared)
  int N, Ns;                // output columns (routed / shared)
  int has_shared;
  int spread_shared;        // shared-expert tiles spread through the schedule (else last)
};

// Workgroups of a persistent launch: one per CU, rounded up to a multiple of
// the XCD count.
int persistent_grid();

// The LDS-tiled kernel: 256 x 256 tiles (gate/up: 128 output columns), bf16
// weights, K and Ks multiples of 64 and at least 256, N and Ns multiples of
// the tile's output columns.
bool lds_gemm_fits(int mode, const GemmArgs& a);
hipError_t launch_lds_gemm(int mode, const GemmArgs& a, hipStream_t st);

}  // namespace moe
