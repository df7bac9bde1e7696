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

template <typename E>
__global__ __launch_bounds__(256) void k_combine(int T, int K, int d, int R,
                                                 const E* __restrict__ y_perm,
                                                 const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ gate,
                                                 const E* __restrict__ shared, E* __restrict__ y) {
  const int t = blockIdx.x;
  const int nvec = d / 8;
  for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
    float acc[8];
    if (shared) {
      Vec8Io<E>::load(shared + (size_t)t * d + c * 8, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      const int row = pair_row[(size_t)t * K + k];
      if (row < 0 || row >= R) continue;
      const float g = gate[(size_t)t * K + k];
      float v[8];
      Vec8Io<E>::load(y_perm + (size_t)row * d + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    Vec8Io<E>::store(y + (size_t)t * d + c * 8, acc);
  }
}

hipError_t launch_combine(int dtype, int T, int K, int d, const void* y_perm,
                          const int32_t* pair_row, const float* gate, const void* shared,
                          void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int R = T * K;
  const int threads = (d / 8) >= 256 ? 256 : 64;
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine<bf16>, dim3(T), dim3(threads), 0, st, T, K, d, R,
                       (const bf16*)y_perm, pair_row, gate, (const bf16*)shared, (bf16*)y);
  else
    hipLaunchKernelGGL(k_combine<float>, dim3(T), dim3(threads), 0, st, T, K, d, R,
                       (const float*)y_perm, pair_row, gate, (const float*)shared, (float*)y);
  return hipGetLastError();
}

}  // namespace moge
