// Permutation of the (token, slot) pairs into expert-contiguous order.
//
// Rows are sorted by expert, then by token, so the result is unique and the
// kernels below reproduce it bit for bit without ordered atomics:
//   1. k_block_hist: per 64-token block, how many pairs go to each expert
//      (popcounts of wave ballots; integer counts, no atomics);
//   2. k_scan: per expert, exclusive prefix over blocks, then over experts ->
//      counts, offsets, per-group loads (every group load equals T*K', the zero
//      imbalance the grouped routing guarantees: TechWalker page, section 一);
//   3. k_scatter: inside a block, the rank of a token among the block's tokens
//      that chose the same expert is a popcount of a wave ballot, so rows come
//      out in token order.
#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

// The set of experts token t chose (entries outside [0, N) and repeats ignored;
// moge_route never produces either).
__device__ __forceinline__ void chosen_set(const int32_t* __restrict__ idx, int t, int K, int N,
                                           bool valid, uint64_t (&chosen)[4]) {
  chosen[0] = chosen[1] = chosen[2] = chosen[3] = 0ull;
  if (!valid) return;
  for (int k = 0; k < K; ++k) {
    const int e = idx[(size_t)t * K + k];
    if ((unsigned)e < (unsigned)N) chosen[e >> 6] |= 1ull << (e & 63);
  }
}

__global__ __launch_bounds__(kPermTokens) void k_block_hist(const int32_t* __restrict__ idx,
                                                            int T, int K, int N,
                                                            int32_t* __restrict__ blk_cnt) {
  const int l = threadIdx.x;
  const int t = blockIdx.x * kPermTokens + l;
  uint64_t chosen[4];
  chosen_set(idx, t, K, N, t < T, chosen);
  int32_t* out = blk_cnt + (size_t)blockIdx.x * N;
  for (int e = 0; e < N; ++e) {
    const uint64_t m = __ballot((chosen[e >> 6] >> (e & 63)) & 1ull);
    if (l == 0) out[e] = __popcll(m);
  }
}

__global__ __launch_bounds__(256) void k_scan(const int32_t* __restrict__ blk_cnt, int nblk,
                                              int N, int M, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ group_counts,
                                              int32_t* __restrict__ blk_base) {
  __shared__ int s_cnt[256];
  const int e = threadIdx.x;
  if (e < N) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      blk_base[(size_t)b * N + e] = run;
      run += blk_cnt[(size_t)b * N + e];
    }
    counts[e] = run;
    s_cnt[e] = run;
  }
  __syncthreads();
  if (e == 0) {
    int acc = 0;
    for (int q = 0; q < N; ++q) {
      offsets[q] = acc;
      acc += s_cnt[q];
    }
    offsets[N] = acc;
  }
  const int G = N / M;
  for (int g = e; g < M; g += 256) {
    int s = 0;
    for (int q = 0; q < G; ++q) s += s_cnt[g * G + q];
    group_counts[g] = s;
  }
}

__global__ __launch_bounds__(kPermTokens) void k_scatter(const int32_t* __restrict__ idx, int T,
                                                         int K, int N,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ blk_base,
                                                         int32_t* __restrict__ sorted_pair,
                                                         int32_t* __restrict__ pair_row) {
  const int l = threadIdx.x;
  const int t = blockIdx.x * kPermTokens + l;
  const bool valid = t < T;
  uint64_t chosen[4];
  chosen_set(idx, t, K, N, valid, chosen);
  // slots that get no row (invalid or repeated expert) keep pair_row = -1
  if (valid)
    for (int k = 0; k < K; ++k) pair_row[(size_t)t * K + k] = -1;
  const uint64_t lt = lanemask_lt();
  const int32_t* base = blk_base + (size_t)blockIdx.x * N;
  for (int e = 0; e < N; ++e) {
    const bool has = (chosen[e >> 6] >> (e & 63)) & 1ull;
    const uint64_t m = __ballot(has);
    if (m == 0ull) continue;
    if (has) {
      int slot = 0;
      while (idx[(size_t)t * K + slot] != e) ++slot;
      const int row = offsets[e] + base[e] + __popcll(m & lt);
      sorted_pair[row] = t * K + slot;
      pair_row[(size_t)t * K + slot] = row;
    }
  }
}

hipError_t launch_permute(const int32_t* idx, int T, int K, int N, int M, int32_t* blk_cnt,
                          int32_t* blk_base, int32_t* counts, int32_t* offsets,
                          int32_t* group_counts, int32_t* sorted_pair, int32_t* pair_row,
                          hipStream_t st) {
  const int nblk = perm_blocks(T);
  hipLaunchKernelGGL(k_block_hist, dim3(nblk), dim3(kPermTokens), 0, st, idx, T, K, N, blk_cnt);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(256), 0, st, blk_cnt, nblk, N, M, counts, offsets,
                     group_counts, blk_base);
  hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(kPermTokens), 0, st, idx, T, K, N, offsets,
                     blk_base, sorted_pair, pair_row);
  return hipGetLastError();
}

// x_perm[row] = x[sorted_pair[row] / K]: one wave per row, 16-byte vectors.
__global__ __launch_bounds__(256) void k_gather_rows(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_pair,
                                                     const int32_t* __restrict__ offsets_end,
                                                     int R, int K, int vec_per_row,
                                                     u32x4* __restrict__ x_perm) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R || row >= *offsets_end) return;
  const int t = sorted_pair[row] / K;
  const u32x4* src = x + (size_t)t * vec_per_row;
  u32x4* dst = x_perm + (size_t)row * vec_per_row;
  for (int v = threadIdx.x & 63; v < vec_per_row; v += 64) dst[v] = src[v];
}

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* sorted_pair,
                              const int32_t* offsets_end, int R, int K, int d, void* x_perm,
                              hipStream_t st) {
  const int vec = d * (dtype == 1 ? 2 : 4) / 16;
  hipLaunchKernelGGL(k_gather_rows, dim3((R + 3) / 4), dim3(256), 0, st, (const u32x4*)x,
                     sorted_pair, offsets_end, R, K, vec, (u32x4*)x_perm);
  return hipGetLastError();
}

}  // namespace moge
