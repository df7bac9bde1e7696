// Gate-weighted combine back to token order:
//   y[t] = shared[t] + sum_k gate[t,k] * y_perm[pair_row[t*K + k]]
// in float32, slots in order k = 0..K-1 (deterministic), rounded once.
// Slots without a row (pair_row < 0, only for invalid routing input) add nothing.
#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

template <typename E> struct Vec8Io;
template <> struct Vec8Io<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float (&v)[8]) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(b[i]);
  }
  static __device__ __forceinline__ void store(bf16* p, const float (&v)[8]) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = static_cast<bf16>(v[i]);
    *reinterpret_cast<bf16x8*>(p) = b;
  }
};
template <> struct Vec8Io<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[i + 4] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

// grid (T, ceil(d / 512)); thread = 8 consecutive features of one token.  The
// slot loop is unrolled by 8 so the K row loads of a token are in flight together;
// the additions still run in slot order.
template <typename E>
__global__ __launch_bounds__(64) void k_combine(int T, int K, int d, int R,
                                                const E* __restrict__ y_perm,
                                                const int32_t* __restrict__ pair_row,
                                                const float* __restrict__ gate,
                                                const E* __restrict__ shared, E* __restrict__ y) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 64 + threadIdx.x;
  if (c >= d / 8) return;
  float acc[8];
  if (shared) {
    Vec8Io<E>::load(shared + (size_t)t * d + c * 8, acc);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  for (int k0 = 0; k0 < K; k0 += 8) {
    int rows[8];
    float g[8], v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j;
      rows[j] = k < K ? pair_row[(size_t)t * K + k] : -1;
      g[j] = k < K ? gate[(size_t)t * K + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] >= 0 && rows[j] < R) {
        Vec8Io<E>::load(y_perm + (size_t)rows[j] * d + c * 8, v[j]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K && rows[j] >= 0 && rows[j] < R) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[j], v[j][i], acc[i]);
      }
  }
  Vec8Io<E>::store(y + (size_t)t * d + c * 8, acc);
}

hipError_t launch_combine(int dtype, int T, int K, int d, const void* y_perm,
                          const int32_t* pair_row, const float* gate, const void* shared,
                          void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int R = T * K;
  dim3 grid(T, (d / 8 + 63) / 64);
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine<bf16>, grid, dim3(64), 0, st, T, K, d, R, (const bf16*)y_perm,
                       pair_row, gate, (const bf16*)shared, (bf16*)y);
  else
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(64), 0, st, T, K, d, R, (const float*)y_perm,
                       pair_row, gate, (const float*)shared, (float*)y);
  return hipGetLastError();
}

}  // namespace moge
