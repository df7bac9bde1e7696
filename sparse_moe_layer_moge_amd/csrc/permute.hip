// Permutation of the (token, slot) pairs into expert-contiguous order.
//
// Rows are sorted by expert, then by token, so the result is unique and the
// kernels below reproduce it bit for bit without ordered atomics.  Tokens are
// handled in chunks of 64, one token per lane:
//   1. per chunk and expert, the mask of the chunk's tokens that chose the expert
//      (built with LDS atomic ORs, one per slot) and its popcount;
//   2. per expert, an exclusive prefix over chunks, then over experts -> counts,
//      offsets and per-group loads (every group load equals T*K', the zero
//      imbalance the grouped routing guarantees: TechWalker page, section 一);
//   3. per chunk, the masks again; the rank of a token among the chunk's
//      tokens that chose expert e is popcount(mask_e & lanes-below-me), so rows
//      come out in token order.
// Small batches run in one workgroup (one launch, all counts in LDS); larger ones
// use a three-kernel version with the same arithmetic, parallel over chunks.
#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

constexpr int kSmallWaves = 16;  // waves of the single-workgroup kernel
constexpr int kSmallChunks = 8;  // chunks up to which it is used (T <= 512): beyond
                                 // that the chunk-parallel kernels finish sooner
constexpr int kSmallIdxCache = 4096;  // slot indices (T * K) it stages in LDS

// f(k, e) for every slot k of token t, in slot order.  The slot indices are
// loaded 8 at a time before any is used, so a token's loads overlap instead of
// paying one memory latency each.
template <typename F>
__device__ __forceinline__ void for_each_slot(const int32_t* idx, int t, int K, F&& f) {
  const int32_t* p = idx + (size_t)t * K;
  for (int k0 = 0; k0 < K; k0 += 8) {
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (k0 + j < K) ? p[k0 + j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < K) f(k0 + j, e[j]);
  }
}

// whether expert e is in a 256-bit set
__device__ __forceinline__ bool in_set(const uint64_t (&s)[4], int e) {
  return (s[e >> 6] >> (e & 63)) & 1ull;
}

// bit l of masks[e] is set when the token of lane l chose expert e (one wave per
// chunk; masks zeroed before).  LDS atomic ORs, one per slot: the result does not
// depend on their order, and an expert repeated in a token sets its bit once.
__device__ __forceinline__ void or_masks(const int32_t* idx, int t, int K, int N, bool valid,
                                         uint64_t* masks) {
  if (!valid) return;
  const int l = threadIdx.x & 63;
  for_each_slot(idx, t, K, [&](int, int e) {
    if ((unsigned)e < (unsigned)N) atomicOr(&masks[e], 1ull << l);
  });
}

// rows of one chunk's pairs: row = offsets[e] + base[e] + rank in chunk; slots
// without a row (invalid or repeated expert) get pair_row = -1
__device__ __forceinline__ void chunk_scatter(const int32_t* __restrict__ idx, int t, int K,
                                              int N, bool valid, const int32_t* offsets,
                                              const int32_t* base, const uint64_t* masks,
                                              int32_t* __restrict__ sorted_pair,
                                              int32_t* __restrict__ pair_row) {
  if (!valid) return;
  const uint64_t lt = lanemask_lt();
  uint64_t seen[4] = {0ull, 0ull, 0ull, 0ull};
  for_each_slot(idx, t, K, [&](int k, int e) {
    int row = -1;
    if ((unsigned)e < (unsigned)N && !in_set(seen, e)) {
      seen[e >> 6] |= 1ull << (e & 63);
      row = offsets[e] + base[e] + __popcll(masks[e] & lt);
      sorted_pair[row] = t * K + k;
    }
    pair_row[(size_t)t * K + k] = row;
  });
}

// inclusive prefix sum across the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v) { return wave_scan_add(v); }

// offsets[e] = exclusive prefix of counts over experts (N <= 256, one wave: lane l
// owns experts 4l .. 4l+3); the total lands in off[N]
__device__ __forceinline__ void expert_offsets(const int32_t* cnt, int N, int32_t* off) {
  const int l = threadIdx.x & 63;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * l + i;
    v[i] = e < N ? cnt[e] : 0;
    s += v[i];
  }
  const int incl = wave_incl_scan(s);
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * l + i;
    if (e < N) off[e] = run;
    run += v[i];
  }
  if (l == 63) off[N] = incl;
}

// ---------------------------------------------------------------------------
// single workgroup: T <= 64 * kSmallChunks.  The masks are built with LDS atomic
// ORs (one wave per chunk; a wave ballot per expert and chunk, as before, took
// 8 us of the kernel's 15 at T=456), the counts and the scatter are split over
// every wave by (chunk, expert) and (chunk, slot).  kCached: the slot
// indices (T * K <= kSmallIdxCache) are copied to LDS first, so that the scatter's
// reads of them (several units per wave, each a dependent read) cost LDS latency.
// ---------------------------------------------------------------------------
template <bool kCached>
__global__ __launch_bounds__(64 * kSmallWaves) void k_permute_small(
    const int32_t* __restrict__ idx_g, int T, int K, int N, int M, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ group_counts,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
  __shared__ uint64_t s_mask[kSmallChunks][256];  // tokens of chunk c that chose e
  __shared__ int32_t s_base[kSmallChunks][256];   // those tokens in chunks before c
  __shared__ int32_t s_cnt[256];
  __shared__ int32_t s_off[257];
  __shared__ int32_t s_idx[kCached ? kSmallIdxCache : 1];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nchunks = (T + 63) / 64;
  const int32_t* idx = idx_g;
  if constexpr (kCached) {
    // every load goes out before the first store, so the copy costs one memory
    // latency instead of one per pass over the workgroup
    constexpr int kPasses = (kSmallIdxCache + 64 * kSmallWaves - 1) / (64 * kSmallWaves);
    int v[kPasses];
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const int i = threadIdx.x + j * 64 * kSmallWaves;
      v[j] = i < T * K ? idx_g[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const int i = threadIdx.x + j * 64 * kSmallWaves;
      if (i < T * K) s_idx[i] = v[j];
    }
    __syncthreads();
    idx = s_idx;
  }

  // masks: bit l of s_mask[c][e] is set when token 64 c + l chose expert e.  Each
  // chunk's wave ORs its tokens' bits into LDS (one atomic per slot; OR does not
  // depend on the order), instead of one ballot per expert and chunk
  for (int i = threadIdx.x; i < nchunks * N; i += blockDim.x) s_mask[i / N][i % N] = 0ull;
  __syncthreads();
  if (w < nchunks) or_masks(idx, w * 64 + l, K, N, w * 64 + l < T, s_mask[w]);
  __syncthreads();
  // per-chunk counts (with one chunk, the totals: nothing comes before it)
  for (int i = threadIdx.x; i < nchunks * N; i += blockDim.x) {
    const int c = i / N, e = i - c * N;
    const int n = __popcll(s_mask[c][e]);
    if (nchunks == 1) {
      s_base[0][e] = 0;
      s_cnt[e] = n;
      counts[e] = n;
    } else {
      s_base[c][e] = n;
    }
  }
  __syncthreads();
  if (nchunks > 1) {
    // per expert: exclusive prefix over the chunks (lane = chunk), total = count
    for (int e = w; e < N; e += kSmallWaves) {
      const int v = l < nchunks ? s_base[l][e] : 0;
      const int incl = wave_incl_scan(v);
      if (l < nchunks) s_base[l][e] = incl - v;
      if (l == 63) {
        s_cnt[e] = incl;
        counts[e] = incl;
      }
    }
    __syncthreads();
  }
  if (w == 0) expert_offsets(s_cnt, N, s_off);
  __syncthreads();
  for (int e = threadIdx.x; e <= N; e += blockDim.x) offsets[e] = s_off[e];
  const int G = N / M;
  for (int g = threadIdx.x; g < M; g += blockDim.x) group_counts[g] = s_off[(g + 1) * G] - s_off[g * G];

  // scatter: unit (chunk c, slot k); lane = token.  row = offset of the expert +
  // its tokens in earlier chunks + its tokens earlier in this chunk.  A slot whose
  // expert is out of range or repeats an earlier slot of the token gets no row.
  const uint64_t lt = lanemask_lt();
  for (int u = w; u < nchunks * K; u += kSmallWaves) {
    const int c = u / K, k = u - c * K, t = c * 64 + l;
    if (t >= T) continue;
    const int32_t* p = idx + (size_t)t * K;
    const int e = p[k];
    bool keep = (unsigned)e < (unsigned)N;
    // the earlier slots, loaded 8 at a time before any is compared
    for (int j0 = 0; j0 < k; j0 += 8) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = j0 + j < k ? p[j0 + j] : -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) keep = keep && v[j] != e;
    }
    int row = -1;
    if (keep) {
      row = s_off[e] + s_base[c][e] + __popcll(s_mask[c][e] & lt);
      sorted_pair[row] = t * K + k;
    }
    pair_row[(size_t)t * K + k] = row;
  }
}

// ---------------------------------------------------------------------------
// large batches: one wave per chunk, three launches
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_chunk_hist(const int32_t* __restrict__ idx, int T, int K,
                                                   int N, int32_t* __restrict__ blk_cnt) {
  __shared__ uint64_t s_mask[256];
  const int l = threadIdx.x;
  const int t = blockIdx.x * 64 + l;
  for (int e = l; e < N; e += 64) s_mask[e] = 0ull;
  __syncthreads();
  or_masks(idx, t, K, N, t < T, s_mask);
  __syncthreads();
  for (int e = l; e < N; e += 64) blk_cnt[(size_t)blockIdx.x * N + e] = __popcll(s_mask[e]);
}

// one workgroup per expert: exclusive prefix of its chunk counts, and its total
__global__ __launch_bounds__(256) void k_scan_chunks(const int32_t* __restrict__ blk_cnt, int nblk,
                                                     int N, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ blk_base) {
  __shared__ int s_sum[4];
  const int e = blockIdx.x;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int v = b < nblk ? blk_cnt[(size_t)b * N + e] : 0;
    const int incl = wave_incl_scan(v);
    if (l == 63) s_sum[w] = incl;
    __syncthreads();
    int before = carry;
    for (int q = 0; q < w; ++q) before += s_sum[q];
    if (b < nblk) blk_base[(size_t)b * N + e] = before + incl - v;
    carry += s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

__global__ __launch_bounds__(64) void k_chunk_scatter(const int32_t* __restrict__ idx, int T,
                                                      int K, int N, int M,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ blk_base,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ group_counts,
                                                      int32_t* __restrict__ sorted_pair,
                                                      int32_t* __restrict__ pair_row) {
  __shared__ uint64_t s_mask[256];
  __shared__ int32_t s_off[257];
  __shared__ int32_t s_base[256];
  const int l = threadIdx.x;
  const int t = blockIdx.x * 64 + l;
  // expert offsets from the totals (every workgroup; the first one publishes them)
  expert_offsets(counts, N, s_off);
  for (int e = l; e < N; e += 64) {
    s_base[e] = blk_base[(size_t)blockIdx.x * N + e];
    s_mask[e] = 0ull;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = l; e <= N; e += 64) offsets[e] = s_off[e];
    const int G = N / M;
    for (int g = l; g < M; g += 64) group_counts[g] = s_off[(g + 1) * G] - s_off[g * G];
  }
  or_masks(idx, t, K, N, t < T, s_mask);
  __syncthreads();
  chunk_scatter(idx, t, K, N, t < T, s_off, s_base, s_mask, sorted_pair, pair_row);
}

hipError_t launch_permute(const int32_t* idx, int T, int K, int N, int M, int32_t* blk_cnt,
                          int32_t* blk_base, int32_t* counts, int32_t* offsets,
                          int32_t* group_counts, int32_t* sorted_pair, int32_t* pair_row,
                          hipStream_t st) {
  const int nblk = perm_blocks(T);
  if (nblk <= kSmallChunks) {
    if ((long long)T * K <= kSmallIdxCache)
      hipLaunchKernelGGL(k_permute_small<true>, dim3(1), dim3(64 * kSmallWaves), 0, st, idx, T, K,
                         N, M, counts, offsets, group_counts, sorted_pair, pair_row);
    else
      hipLaunchKernelGGL(k_permute_small<false>, dim3(1), dim3(64 * kSmallWaves), 0, st, idx, T,
                         K, N, M, counts, offsets, group_counts, sorted_pair, pair_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_chunk_hist, dim3(nblk), dim3(64), 0, st, idx, T, K, N, blk_cnt);
  hipLaunchKernelGGL(k_scan_chunks, dim3(N), dim3(256), 0, st, blk_cnt, nblk, N, counts, blk_base);
  hipLaunchKernelGGL(k_chunk_scatter, dim3(nblk), dim3(64), 0, st, idx, T, K, N, M, counts,
                     blk_base, offsets, group_counts, sorted_pair, pair_row);
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
