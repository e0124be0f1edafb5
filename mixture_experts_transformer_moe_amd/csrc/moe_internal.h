// Internal declarations shared by the HIP translation units of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- types
typedef uint16_t bf16_t;   // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 by gfx950's v_cvt_pk_bf16_f32: round to nearest, ties to
// even (the default rounding mode); NaN stays NaN, overflow goes to inf.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.0f));
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

// --------------------------------------------------------------- launchers
// All return hipSuccess or the launch error; they assume validated arguments.
// mask: null, or one byte per token (0 = padding: not routed, expert -1)
hipError_t launch_route_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wr,
                             const float* bias, const uint8_t* mask, float* logits, int32_t* idx,
                             float* w, hipStream_t st);
hipError_t launch_route_f32(const moe_shape& s, const float* x, const float* wr,
                            const float* bias, const uint8_t* mask, float* logits, int32_t* idx,
                            float* w, hipStream_t st);

size_t permute_workspace_bytes(const moe_shape& s);
// the device-resident scratch of moe_permute_static: its size, and its address
// on the current device (looked up once per device)
size_t static_scratch_bytes();
hipError_t static_scratch(void** out);
hipError_t launch_permute(const moe_shape& s, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* slot_of,
                          void* x_perm, void* workspace, hipStream_t st);

hipError_t launch_gate_up_bf16(const moe_shape& s, const bf16_t* x_perm,
                               const int32_t* sorted_token, const bf16_t* x,
                               const int32_t* offsets, const bf16_t* wgu, const bf16_t* wsgu,
                               bf16_t* h, hipStream_t st);
hipError_t launch_down_bf16(const moe_shape& s, const bf16_t* h, const int32_t* offsets,
                            const bf16_t* wd, const bf16_t* wsd, bf16_t* y_perm,
                            bf16_t* y_shared, hipStream_t st);
hipError_t launch_shared_ffn_bf16(const moe_shape& s, const bf16_t* x, const bf16_t* wsgu,
                                  const bf16_t* wsd, bf16_t* hs, bf16_t* ys, hipStream_t st);
// training pass (grouped_gemm.hip): pre-activations [g | u] of every routed
// row and of the shared expert; dh = dy W_d; da = [dg | du] [W_g; W_u]; a
// dense product out = a W^T with W packed [N, K]
hipError_t launch_gate_up_pre_bf16(const moe_shape& s, const bf16_t* x_perm,
                                   const int32_t* sorted_token, const bf16_t* x,
                                   const int32_t* offsets, const bf16_t* wgu, const bf16_t* wsgu,
                                   bf16_t* gu, hipStream_t st);
hipError_t launch_dgrad_h_bf16(const moe_shape& s, const bf16_t* dy_perm, const bf16_t* dout,
                               const int32_t* offsets, const bf16_t* wd_t, const bf16_t* wsd_t,
                               bf16_t* dh, hipStream_t st);
hipError_t launch_dgrad_x_bf16(const moe_shape& s, const bf16_t* dgu, const int32_t* offsets,
                               const bf16_t* wgu_t, const bf16_t* wsgu_t, bf16_t* dx_perm,
                               bf16_t* dx_shared, hipStream_t st);
hipError_t launch_dense_bf16(int rows, int K, int N, const bf16_t* a_rows, const bf16_t* w_packed,
                             bf16_t* out, hipStream_t st);
hipError_t launch_gate_up_f32(const moe_shape& s, const float* x_perm,
                              const int32_t* sorted_token, const float* x,
                              const int32_t* offsets, const float* wgu, const float* wsgu,
                              float* h, hipStream_t st);
hipError_t launch_down_f32(const moe_shape& s, const float* h, const int32_t* offsets,
                           const float* wd, const float* wsd, float* y_perm, float* y_shared,
                           hipStream_t st);

// Packed [rows x K] weight matrix (moe_pack_weights): block (row / 32, k / 16)
// is 512 contiguous elements, in which lane (row % 32) + 32 ((k % 16) / 8)
// holds elements k % 8 = 0..7; blocks are row-block major.
__host__ __device__ __forceinline__ size_t packed_matrix_elems(int rows, int K) {
  return static_cast<size_t>(rows) * K;
}

__host__ __device__ __forceinline__ size_t packed_offset(int row, int k, int K) {
  const size_t blk = static_cast<size_t>(row >> 5) * (K >> 4) + (k >> 4);
  return blk * 512 + ((row & 31) + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
}

hipError_t launch_quantize_fp8(const void* src, void* dst, float* scales, int64_t count, int rows,
                               int cols, hipStream_t st);
hipError_t launch_gate_up_fp8(const moe_shape& s, const bf16_t* x_perm, const int32_t* sorted_token,
                              const bf16_t* x, const int32_t* offsets, const uint8_t* wgu,
                              const float* sgu, const uint8_t* wsgu, const float* ssgu, bf16_t* h,
                              hipStream_t st);
hipError_t launch_down_fp8(const moe_shape& s, const bf16_t* h, const int32_t* offsets,
                           const uint8_t* wd, const float* sd, const uint8_t* wsd, const float* ssd,
                           bf16_t* y_perm, bf16_t* y_shared, hipStream_t st);
hipError_t launch_pack(const void* src, void* dst, int64_t count, int rows, int cols, int elem,
                       hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                          const int32_t* slot_of, const float* topk_w, void* out,
                          hipStream_t st);

// ---------------------------------------------------------- training pass
hipError_t launch_pack_transposed(const void* src, void* dst, int64_t count, int rows, int cols, int kp,
                                  hipStream_t st);
size_t train_workspace_bytes(const moe_shape& s);
hipError_t launch_swiglu_pre(const moe_shape& s, const bf16_t* gu, const int32_t* offsets, bf16_t* h,
                             hipStream_t st);
hipError_t launch_swiglu_bwd(const moe_shape& s, const bf16_t* dh, const bf16_t* gu,
                             const int32_t* offsets, bf16_t* dgu, hipStream_t st);
hipError_t launch_combine_bwd(const moe_shape& s, const bf16_t* dout, const bf16_t* y_perm,
                              const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w,
                              const float* logits, const float* coef, bf16_t* dy_perm, float* dz,
                              bf16_t* dz16, hipStream_t st);
hipError_t launch_dx_reduce(const moe_shape& s, const bf16_t* dx_perm, const bf16_t* dx_shared,
                            const bf16_t* dx_router, const int32_t* slot_of, bf16_t* dx, hipStream_t st);
hipError_t launch_load_stats(const moe_shape& s, const float* logits, const int32_t* topk_idx,
                             const int32_t* counts, const int32_t* counts_global, float beta, float* f,
                             float* p, float* loss, float* coef, void* ws, hipStream_t st);
hipError_t launch_colsum(const moe_shape& s, const float* m, float* out, void* ws, hipStream_t st);
hipError_t launch_wgrad(const moe_shape& s, const bf16_t* x, const int32_t* sorted_token,
                        const bf16_t* x_perm, const bf16_t* dgu, const bf16_t* dy, const bf16_t* h,
                        const bf16_t* dout, const bf16_t* dz16, const int32_t* offsets, bf16_t* dwgu,
                        bf16_t* dwd, bf16_t* dwsgu, bf16_t* dwsd, float* dwr, hipStream_t st);

}  // namespace moe
