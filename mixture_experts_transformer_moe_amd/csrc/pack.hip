// Weight packing into MFMA fragment order (one pass, at weight-load time), and
// the FP8 (E4M3, per-row scale) quantisation of bf16 weights into the same
// kind of order.
//
// A matrix W [rows x cols] (row-major, rows % 32 == 0, cols % 16 == 0) becomes
// blocks of 32 rows x 16 columns, row-block major then column-block; inside a
// block, lane l = (r % 32) + 32 ((c % 16) / 8) holds its 8 elements
// c % 8 = 0..7 contiguously.  That is exactly the operand one wave feeds to a
// 32x32x16 MFMA for one 32-row block and one 16-wide K step, so a wave streams
// a block row with whole 1 KB (bf16) loads.  The permutation keeps the size.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                   int64_t count, int rows, int cols) {
  const int cb = cols >> 4;                                          // column blocks
  const int64_t per_mat = static_cast<int64_t>(rows) * cols / 8;     // 8-element groups
  const int64_t groups = count * per_mat;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; gi < groups;
       gi += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t mi = gi / per_mat;
    const int64_t in = gi - mi * per_mat;
    const int64_t blk = in >> 6;
    const int lane = static_cast<int>(in & 63);
    const int nb = static_cast<int>(blk / cb), kb = static_cast<int>(blk % cb);
    const int row = nb * 32 + (lane & 31);
    const int col = kb * 16 + 8 * (lane >> 5);
    const T* s = src + (mi * rows + row) * static_cast<int64_t>(cols) + col;
    T* d = dst + gi * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = s[e];
  }
}

// Transposed packing for the backward products: matrix i of src [count, rows,
// cols] becomes its transpose [cols, kp] in the packed order above, with
// columns k >= rows of the transpose zero (kp >= rows, kp % 16 == 0).  Lanes
// of a wave read consecutive source columns of the same source row.
__global__ __launch_bounds__(256) void pack_transposed_kernel(const uint16_t* __restrict__ src,
                                                              uint16_t* __restrict__ dst,
                                                              int64_t count, int rows, int cols,
                                                              int kp) {
  const int cb = kp >> 4;                                            // column blocks of the transpose
  const int64_t per_mat = static_cast<int64_t>(cols) * kp / 8;       // 8-element groups
  const int64_t groups = count * per_mat;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; gi < groups;
       gi += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t mi = gi / per_mat;
    const int64_t in = gi - mi * per_mat;
    const int64_t blk = in >> 6;
    const int lane = static_cast<int>(in & 63);
    const int nb = static_cast<int>(blk / cb), kb = static_cast<int>(blk % cb);
    const int trow = nb * 32 + (lane & 31);                          // a source column
    const int tcol = kb * 16 + 8 * (lane >> 5);                      // source rows tcol..tcol+7
    const uint16_t* s = src + mi * rows * static_cast<int64_t>(cols) + trow;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tcol + e < rows ? s[static_cast<int64_t>(tcol + e) * cols] : 0;
    uint16_t* d = dst + gi * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = v[e];
  }
}

// E4M3 code of a finite fp32 value: round to nearest, ties to even, magnitudes
// past 448 saturating to 448 (OCP FP8 E4M3: bias 7, subnormals below 2^-6, no
// infinities, 0x7F / 0xFF are NaN and never produced).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t u = bits & 0x7fffffffu;
  uint32_t mag;
  if (u >= 0x43E80000u) {               // >= 464, midway 448 and the (absent) 480
    mag = 0x7Eu;
  } else if (u < 0x3C800000u) {         // below 2^-6: multiples of 2^-9
    mag = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(u) * 512.0f));   // 0..8, exact scaling
  } else {                              // normal: 3 mantissa bits, ties to even on bit 20
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    mag = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  }
  return sign | mag;
}

// One wave per matrix row: amax, scale = amax / 448 (1 for a zero row), then
// the codes of w / scale, 8 per lane and store, in the FP8 fragment order: the
// 8 columns c0..c0+7 (c0 % 8 == 0) of row r sit at byte
//   ((r / 32) (cols / 32) + c0 / 32) 1024 + ((r % 32) + 32 ((c0 / 8) % 2)) 16 + ((c0 / 16) % 2) 8,
// i.e. 32 x 32 blocks of 1 KB in which lane l's 16 bytes are its 8 codes of
// two consecutive 16-wide K steps.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst,
                                                           float* __restrict__ scales, int64_t nrows,
                                                           int rows, int cols) {
  const int lane = threadIdx.x & 63;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gr >= nrows) return;
  const int64_t mi = gr / rows;
  const int r = static_cast<int>(gr - mi * rows);
  const uint16_t* row = src + gr * cols;
  float amax = 0.0f;
  for (int c0 = 8 * lane; c0 < cols; c0 += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[i] << 16)), fabsf(__uint_as_float(w[i] & 0xffff0000u))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) scales[gr] = scale;
  uint8_t* mat = dst + mi * static_cast<int64_t>(rows) * cols;
  for (int c0 = 8 * lane; c0 < cols; c0 += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t q[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = e4m3_rne(__uint_as_float(w[i] << 16) / scale);
      const uint32_t hi = e4m3_rne(__uint_as_float(w[i] & 0xffff0000u) / scale);
      q[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    const int64_t off = (static_cast<int64_t>(r >> 5) * (cols >> 5) + (c0 >> 5)) * 1024 +
                        ((r & 31) + 32 * ((c0 >> 3) & 1)) * 16 + ((c0 >> 4) & 1) * 8;
    *reinterpret_cast<uint2*>(mat + off) = make_uint2(q[0], q[1]);
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* src, void* dst, float* scales, int64_t count, int rows,
                               int cols, hipStream_t st) {
  const int64_t nrows = count * rows;
  if (nrows == 0 || cols == 0) return hipSuccess;
  const int64_t blocks = (nrows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  quantize_fp8_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(
      static_cast<const uint16_t*>(src), static_cast<uint8_t*>(dst), scales, nrows, rows, cols);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, void* dst, int64_t count, int rows, int cols, int elem,
                       hipStream_t st) {
  const int64_t groups = count * static_cast<int64_t>(rows) * cols / 8;
  if (groups == 0) return hipSuccess;
  const int64_t want = (groups + 255) / 256;
  const int blocks = static_cast<int>(want < 65536 ? want : 65536);
  if (elem == 2)
    pack_kernel<uint16_t><<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(src),
                                                  static_cast<uint16_t*>(dst), count, rows, cols);
  else
    pack_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(src), static_cast<float*>(dst),
                                               count, rows, cols);
  return hipGetLastError();
}

hipError_t launch_pack_transposed(const void* src, void* dst, int64_t count, int rows, int cols, int kp,
                                  hipStream_t st) {
  const int64_t groups = count * static_cast<int64_t>(cols) * kp / 8;
  if (groups == 0) return hipSuccess;
  const int64_t want = (groups + 255) / 256;
  const int blocks = static_cast<int>(want < 65536 ? want : 65536);
  pack_transposed_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(src),
                                                 static_cast<uint16_t*>(dst), count, rows, cols, kp);
  return hipGetLastError();
}

}  // namespace moe
