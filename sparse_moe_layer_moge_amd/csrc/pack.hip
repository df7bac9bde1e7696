// moge_pack_weights: copy row-major expert weights into the packed fragment
// layout (packed_layout.hpp).  A pure permutation of 8-element chunks.
#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "packed_layout.hpp"

namespace moge {

// One thread per 8-element lane chunk of the destination.
//   gate/up mode (src1 != nullptr): expert has `rows` rows in each of src0/src1,
//     blocks of 16 rows, tile 0 from src0, tile 1 from src1;
//   down mode (src1 == nullptr): expert has `rows` rows in src0, blocks of 32 rows,
//     tile t covers rows 32b + 16t .. 32b + 16t + 15.
template <typename E>
__global__ __launch_bounds__(256) void k_pack(const E* __restrict__ src0,
                                              const E* __restrict__ src1, int n_exp, int rows,
                                              int K, E* __restrict__ dst) {
  const int nsteps = K / 32;
  const bool gu = src1 != nullptr;
  const int block_rows = gu ? 16 : 32;
  const int nblocks = rows / block_rows;
  const size_t chunks_per_expert = (size_t)(gu ? 2 * rows : rows) * K / 8;
  const size_t total = chunks_per_expert * n_exp;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t tile = c >> 6;
    const int t = (int)(tile & 1);
    tile >>= 1;
    const int s = (int)(tile % nsteps);
    tile /= nsteps;
    const int b = (int)(tile % nblocks);
    const int e = (int)(tile / nblocks);
    const E* src = (gu && t == 1) ? src1 : src0;
    const int row = b * block_rows + (gu ? 0 : 16 * t) + (lane & 15);
    const int k = s * 32 + (lane >> 4) * 8;
    const E* from = src + ((size_t)e * rows + row) * K + k;
    E* to = dst + c * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) to[i] = from[i];
  }
}

hipError_t launch_pack(int dtype, const void* src0, const void* src1, int n_exp, int rows, int K,
                       void* dst, hipStream_t st) {
  const size_t chunks = (size_t)n_exp * (src1 ? 2 * rows : rows) * K / 8;
  if (chunks == 0) return hipSuccess;
  const size_t want = (chunks + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  if (dtype == 1)
    hipLaunchKernelGGL(k_pack<bf16>, dim3(blocks), dim3(256), 0, st, (const bf16*)src0,
                       (const bf16*)src1, n_exp, rows, K, (bf16*)dst);
  else
    hipLaunchKernelGGL(k_pack<float>, dim3(blocks), dim3(256), 0, st, (const float*)src0,
                       (const float*)src1, n_exp, rows, K, (float*)dst);
  return hipGetLastError();
}

}  // namespace moge
