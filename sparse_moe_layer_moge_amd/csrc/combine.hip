// Gate-weighted combine back to token order:
//   y[t] = shared[t] + sum_k gate[t,k] * y_perm[pair_row[t*K + k]]
// in float32, slots in order k = 0..K-1 (deterministic), rounded once.  The shared
// term is either the shared experts' output or the float32 partial sums of its
// split contraction, added in slice order first.
// Slots without a row (pair_row < 0, only for invalid routing input) add nothing.
#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

// bf16 rows are read and written once each (the slot rows, the shared term, y):
// non-temporal accesses (16384 tokens: combine 0.333 -> 0.300 ms)
template <typename E> struct Vec8Io;
template <> struct Vec8Io<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float (&v)[8]) {
    const bf16x8 b = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(b[i]);
  }
  static __device__ __forceinline__ void store(bf16* p, const float (&v)[8]) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = static_cast<bf16>(v[i]);
    __builtin_nontemporal_store(b, reinterpret_cast<bf16x8*>(p));
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

// grid (T, ceil(d / 512)); thread = 8 consecutive features of one token.  Loads go
// out in batches so that a thread waits for memory about twice, not once per
// term: the first 8 slots' rows and gates together with every partial slice of
// the shared term, then those slots' y_perm rows (with the next 8 slots' rows
// and gates).  The additions still run in slice order, then slot order.
template <typename E>
__global__ __launch_bounds__(64) void k_combine(int T, int K, int d, int R,
                                                const E* __restrict__ y_perm,
                                                const int32_t* __restrict__ pair_row,
                                                const float* __restrict__ gate,
                                                const E* __restrict__ shared,
                                                const float* __restrict__ shared_part,
                                                int n_part, E* __restrict__ y) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * 64 + threadIdx.x;
  if (c >= d / 8) return;
  int rows[8];
  float g[8];
  // (slots past K read slot K - 1 and are dropped: no branch per load, so the
  // 16 scalar loads go out together)
  auto load_slots = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = min(k0 + j, K - 1);
      rows[j] = pair_row[(size_t)t * K + k];
      g[j] = gate[(size_t)t * K + k];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j >= K) rows[j] = -1;
  };
  load_slots(0);
  float acc[8];
  if (shared_part) {
    float sp[kMaxSlices][8];
#pragma unroll
    for (int p = 0; p < kMaxSlices; ++p)
      if (p < n_part) Vec8Io<float>::load(shared_part + ((size_t)p * T + t) * d + c * 8, sp[p]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = sp[0][i];
#pragma unroll
    for (int p = 1; p < kMaxSlices; ++p)
      if (p < n_part) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += sp[p][i];
      }
  } else if (shared) {
    Vec8Io<E>::load(shared + (size_t)t * d + c * 8, acc);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  for (int k0 = 0; k0 < K; k0 += 8) {
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] >= 0 && rows[j] < R) {
        Vec8Io<E>::load(y_perm + (size_t)rows[j] * d + c * 8, v[j]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
      }
    }
    int rr[8];
    float gg[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rr[j] = rows[j];
      gg[j] = g[j];
    }
    if (k0 + 8 < K) load_slots(k0 + 8);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K && rr[j] >= 0 && rr[j] < R) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(gg[j], v[j][i], acc[i]);
      }
  }
  Vec8Io<E>::store(y + (size_t)t * d + c * 8, acc);
}

hipError_t launch_combine(int dtype, int T, int K, int d, const void* y_perm,
                          const int32_t* pair_row, const float* gate, const void* shared,
                          const float* shared_part, int n_part, void* y, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (shared_part && (n_part < 1 || n_part > kMaxSlices)) return hipErrorInvalidValue;
  const int R = T * K;
  dim3 grid(T, (d / 8 + 63) / 64);
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine<bf16>, grid, dim3(64), 0, st, T, K, d, R, (const bf16*)y_perm,
                       pair_row, gate, (const bf16*)shared, shared_part, n_part, (bf16*)y);
  else
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(64), 0, st, T, K, d, R, (const float*)y_perm,
                       pair_row, gate, (const float*)shared, shared_part, n_part, (float*)y);
  return hipGetLastError();
}

// H[r, f] = silu(sum_s g[s][r][f]) * sum_s u[s][r][f] (slices in order), rounded to
// bf16 once; g = part, u = part + ksplit * rows * inter.  One thread per 8 features.
__global__ __launch_bounds__(256) void k_swiglu_parts(const float* __restrict__ part, int ksplit,
                                                      int rows, int inter, bf16* __restrict__ h) {
  const size_t n8 = (size_t)rows * inter / 8;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const size_t plane = (size_t)rows * inter;
  const float* up = part + (size_t)ksplit * plane;
  // every slice's loads go out before any is added
  float a[kMaxSlices][8], b[kMaxSlices][8];
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s)
    if (s < ksplit) {
      Vec8Io<float>::load(part + s * plane + i * 8, a[s]);
      Vec8Io<float>::load(up + s * plane + i * 8, b[s]);
    }
  float g[8], u[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    g[j] = a[0][j];
    u[j] = b[0][j];
  }
#pragma unroll
  for (int s = 1; s < kMaxSlices; ++s)
    if (s < ksplit) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        g[j] += a[s][j];
        u[j] += b[s][j];
      }
    }
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = silu(g[j]) * u[j];
  Vec8Io<bf16>::store(h + i * 8, v);
}

hipError_t launch_swiglu_parts(const float* part, int ksplit, int rows, int inter, void* h,
                               hipStream_t st) {
  const size_t n8 = (size_t)rows * inter / 8;
  if (n8 == 0) return hipSuccess;
  if (ksplit < 1 || ksplit > kMaxSlices) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_swiglu_parts, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, part,
                     ksplit, rows, inter, (bf16*)h);
  return hipGetLastError();
}

}  // namespace moge
