// Weight packing into MFMA fragment order (one pass, at weight-load time).
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

}  // namespace

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

}  // namespace moe
