// Router: scores x W_r^T (+b), global softmax over all experts, per-group top-K'.
//
// Grouped routing as the TechWalker page describes it (section 一 创新架构): the
// softmax runs over every routed expert first; then each of the M equal groups
// keeps its own K' best experts, so every group receives the same number of
// (token, expert) pairs.  The Reportify concept page (技术创新细节) states the same:
// each group routes its top-K independently, and the load difference between
// groups is zero.
#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "stream_tile.hpp"

namespace moge {

// ---------------------------------------------------------------------------
// scores: one wave per (16 experts x 16 tokens) tile and contraction split.
// A operand = router weight rows (experts), B operand = token rows; the MFMA
// result D[expert][token] leaves four consecutive experts of one token per lane.
// Splitting the contraction gives the small-T (decode) case enough waves; the
// partial sums are added in a fixed order by the routing kernel.
// ---------------------------------------------------------------------------
template <typename E, int PW>
__global__ __launch_bounds__(64) void k_router_scores(const E* __restrict__ x,
                                                      const E* __restrict__ wr, int T, int d,
                                                      int N, int steps_per_split,
                                                      float* __restrict__ partial) {
  const int l = threadIdx.x;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16, ks = blockIdx.z;
  const int nsteps = d / 32;
  const int s0 = ks * steps_per_split;
  const int n = min(nsteps, s0 + steps_per_split) - s0;
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  if (n > 0) {
    const int ln = l & 15, kq = (l >> 4) * 8;
    const uint32_t base = (uint32_t)((s0 * 32 + kq) * sizeof(E));
    const Rsrc rw[1] = {make_rsrc(wr, (uint64_t)N * d * sizeof(E))};
    const uint32_t vw[1] = {(uint32_t)(min(e0 + ln, N - 1) * d * sizeof(E)) + base};
    const uint32_t vx[1] = {(uint32_t)((size_t)min(t0 + ln, T - 1) * d * sizeof(E)) + base};
    const Rsrc rx = make_rsrc(x, (uint64_t)T * d * sizeof(E));
    if (n >= PW)
      stream_tile<E, 1, 1, PW>(rw, vw, 32 * sizeof(E), rx, vx, n, 0, acc);
    else
      stream_tile<E, 1, 1, 1>(rw, vw, 32 * sizeof(E), rx, vx, n, 0, acc);
  }
  const int t = t0 + (l & 15);
  if (t < T) {
    float* out = partial + ((size_t)ks * T + t) * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + 4 * (l >> 4) + i;
      if (e < N) out[e] = acc[0][0][i];
    }
  }
}

// ---------------------------------------------------------------------------
// scores for large batches (bf16): one workgroup per 128 tokens x 64 experts and
// contraction split, MFMA 32x32x16.  Both operands go through a 4-stage LDS ring
// of 64-element stages, loaded straight into LDS as 128-byte row lines (8 rows per
// wave instruction) with the chunks XOR-swizzled by row, as in the expert tile
// kernels; the router weights are then read from L2 once per workgroup instead of
// once per 16-token wave, and every token row once per expert block.
// ---------------------------------------------------------------------------
constexpr int kRtM = 128;                       // tokens per tile (32 per wave)
constexpr int kRtN = 64;                        // experts per tile
constexpr int kRtStages = 4;
constexpr int kRtLine = 128;                    // bytes of a row per stage (64 bf16)
constexpr int kRtABytes = kRtM * kRtLine;       // 16 KiB
constexpr int kRtStageBytes = (kRtM + kRtN) * kRtLine;
constexpr int kRtMinTokens = 2048;              // below this the wave kernel above is used

typedef __attribute__((address_space(3))) void* RtLdsPtr;

__device__ __forceinline__ void rt_dma16(Rsrc r, uint32_t voff, uint32_t soff, uint32_t m0v) {
  // 64 lanes x 16 bytes into LDS at m0v + 16 * lane; counted with vmcnt by the
  // caller.  M0 is used by nothing else in this kernel.
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}
template <int N> __device__ __forceinline__ void rt_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(256, 1) void k_router_tile(const bf16* __restrict__ x,
                                                        const bf16* __restrict__ wr, int T,
                                                        int d, int N, int stages_per_split,
                                                        float* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) char lds[kRtStages * kRtStageBytes];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRtM, e0 = blockIdx.y * kRtN, ks = blockIdx.z;
  const int nst = d / 64;
  const int s0 = ks * stages_per_split;
  const int n = min(nst, s0 + stages_per_split) - s0;
  f32x16 acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
  if (n > 0) {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(RtLdsPtr)lds);
    const Rsrc xr = make_rsrc(x, (uint64_t)T * d * sizeof(bf16));
    const Rsrc wrr = make_rsrc(wr, (uint64_t)N * d * sizeof(bf16));
    // this wave loads token rows 8 (4 wu + i) + l / 8 and expert rows 8 (2 wu + i) + l / 8
    // of a stage; lane l fetches the chunk that its LDS slot l % 8 holds
    const int lr = l >> 3;
    uint32_t va[4], vb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * wu + i) * 8 + lr;
      const int t = min(t0 + r, T - 1);
      va[i] = (uint32_t)(((size_t)t * d + ((l & 7) ^ ((r >> 1) & 7)) * 8) * sizeof(bf16));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (2 * wu + i) * 8 + lr;
      const int e = min(e0 + r, N - 1);
      vb[i] = (uint32_t)(((size_t)e * d + ((l & 7) ^ ((r >> 1) & 7)) * 8) * sizeof(bf16));
    }
    auto issue = [&](int j, int st) {   // load j (0..5) of this wave for stage st
      const uint32_t base = lds0 + (uint32_t)((st % kRtStages) * kRtStageBytes);
      const uint32_t so = (uint32_t)(s0 + st) * kRtLine;
      if (j < 4)
        rt_dma16(xr, va[j], so, base + (4 * wu + j) * 8 * kRtLine);
      else
        rt_dma16(wrr, vb[j - 4], so, base + kRtABytes + (2 * wu + j - 4) * 8 * kRtLine);
    };
    const int lane_row = (l & 31) * kRtLine;
    const int lswz = ((l & 31) >> 1) & 7;
#pragma unroll
    for (int st = 0; st < kRtStages - 1; ++st)
      if (st < n) {
#pragma unroll
        for (int j = 0; j < 6; ++j) issue(j, st);
      }
    for (int kb = 0; kb < n; ++kb) {
      // this wave's loads of stage kb are in when at most those of the stages
      // kb+1 .. min(kb + 2, n - 1), issued after them, are outstanding
      const int later = min(kRtStages - 2, n - 1 - kb);
      if (later >= 2)
        rt_wait<12>();
      else if (later == 1)
        rt_wait<6>();
      else
        rt_wait<0>();
      asm volatile("s_barrier" ::: "memory");
      const char* A = lds + (kb % kRtStages) * kRtStageBytes;
      const char* B = A + kRtABytes;
      const bool more = kb + kRtStages - 1 < n;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int off = lane_row + (((2 * h + (l >> 5)) ^ lswz) << 4);
        const bf16x8 tf = *reinterpret_cast<const bf16x8*>(A + wu * 32 * kRtLine + off);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8 wf = *reinterpret_cast<const bf16x8*>(B + q * 32 * kRtLine + off);
          acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, tf, acc[q], 0, 0, 0);
          const int m = 2 * h + q;
          if (more && m < 6) issue(m, kb + kRtStages - 1);
        }
      }
    }
  }
  // lane l, register r: expert e0 + 32 q + 8 (r / 4) + 4 (l / 32) + r % 4 of token
  // t0 + 32 w + l % 32
  const int t = t0 + w * 32 + (l & 31);
  if (t < T) {
    float* out = partial + ((size_t)ks * T + t) * N;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = e0 + 32 * q + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (e < N) out[e] = acc[q][r];
      }
  }
}

static bool router_tiles(int dtype, int T, int d) {
  return dtype == 1 && T >= kRtMinTokens && d % 64 == 0;
}

// contraction splits of the router scores (k_route sums at most this many)
constexpr int kMaxRouterSplit = 16;

int router_ksplit(int dtype, int T, int d, int N) {
  if (router_tiles(dtype, T, d)) {
    // about one workgroup per CU, with no empty split
    const int tiles = ((T + kRtM - 1) / kRtM) * ((N + kRtN - 1) / kRtN);
    const int nst = d / 64;
    int ks = 256 / (tiles > 0 ? tiles : 1);
    if (ks < 1) ks = 1;
    if (ks > kMaxRouterSplit) ks = kMaxRouterSplit;
    if (ks > nst) ks = nst;
    const int per = (nst + ks - 1) / ks;
    return (nst + per - 1) / per;
  }
  // enough waves to spread the router weight and x over the CUs at decode sizes
  // (about four per CU: at T=456, 8 slices instead of 4 took the scores from
  // 11.3 to 10.2 us; 16 gained nothing more), few partial sums at prefill sizes
  const int tiles = ((T + 15) / 16) * ((N + 15) / 16);
  const int nsteps = d / 32;
  int ks = 1024 / (tiles > 0 ? tiles : 1);
  if (ks < 1) ks = 1;
  if (ks > kMaxRouterSplit) ks = kMaxRouterSplit;
  if (ks > nsteps) ks = nsteps;
  return ks;
}

hipError_t launch_router_scores(int dtype, const void* x, const void* w_router, int T, int d,
                                int N, int ksplit, float* partial, hipStream_t st) {
  if (router_tiles(dtype, T, d)) {
    const int nst = d / 64;
    const int per = (nst + ksplit - 1) / ksplit;
    dim3 grid((T + kRtM - 1) / kRtM, (N + kRtN - 1) / kRtN, ksplit);
    hipLaunchKernelGGL(k_router_tile, grid, dim3(256), 0, st, (const bf16*)x,
                       (const bf16*)w_router, T, d, N, per, partial);
    return hipGetLastError();
  }
  const int nsteps = d / 32;
  const int per = (nsteps + ksplit - 1) / ksplit;
  dim3 grid((N + 15) / 16, (T + 15) / 16, ksplit);
  if (dtype == 1)
    hipLaunchKernelGGL((k_router_scores<bf16, 4>), grid, dim3(64), 0, st, (const bf16*)x,
                       (const bf16*)w_router, T, d, N, per, partial);
  else
    hipLaunchKernelGGL((k_router_scores<float, 4>), grid, dim3(64), 0, st, (const float*)x,
                       (const float*)w_router, T, d, N, per, partial);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// routing: one wave per token, lane j holds experts j, j+64, j+128, j+192.
// Selection compares float32 scores only (exact); equal scores go to the lower
// expert index because a candidate replaces the current best only when strictly
// greater while experts are visited in increasing index order.
// ---------------------------------------------------------------------------
constexpr int kRouteWaves = 4;

__global__ __launch_bounds__(256) void k_route(const float* __restrict__ partial, int ksplit,
                                               int T, int N, int M, int kp,
                                               const float* __restrict__ bias,
                                               float* __restrict__ logits_out,
                                               float* __restrict__ probs,
                                               int32_t* __restrict__ idx,
                                               float* __restrict__ gate,
                                               int* __restrict__ zero, int n_zero) {
  __shared__ float s_l[kRouteWaves][256];
  __shared__ float s_p[kRouteWaves][256];
  // the layer's work counters for the expert launches that follow
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[i] = 0;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + w;
  const bool valid = t < T;
  const int tt = valid ? t : 0;

  float v[4], ex[4];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l + 64 * j;
    v[j] = -INFINITY;
    if (e < N) {
      // every split's partial is loaded before any is added (one memory latency,
      // not one per batch); start from split 0 (not from 0.f) so a lone -0.0
      // score keeps its sign, and add the splits in increasing order
      float pv[kMaxRouterSplit];
#pragma unroll
      for (int ks = 0; ks < kMaxRouterSplit; ++ks)
        pv[ks] = ks < ksplit ? partial[((size_t)ks * T + tt) * N + e] : 0.f;
      const float b = bias ? bias[e] : 0.f;
      float s = pv[0];
#pragma unroll
      for (int ks = 1; ks < kMaxRouterSplit; ++ks)
        if (ks < ksplit) s += pv[ks];
      if (bias) s += b;
      v[j] = s;
      mx = fmaxf(mx, s);
    }
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l + 64 * j;
    ex[j] = (e < N) ? expf(v[j] - mx) : 0.f;
    sum += ex[j];
  }
  sum = wave_sum(sum);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l + 64 * j;
    if (e < N) {
      const float p = ex[j] / sum;
      s_l[w][e] = v[j];
      s_p[w][e] = p;
      if (valid && logits_out) logits_out[(size_t)t * N + e] = v[j];
      if (valid && probs) probs[(size_t)t * N + e] = p;
    }
  }
  __syncthreads();
  if (!valid) return;
  const int G = N / M, K = M * kp;
  for (int g = l; g < M; g += 64) {
    uint64_t taken[4] = {0ull, 0ull, 0ull, 0ull};
    for (int j = 0; j < kp; ++j) {
      int bi = -1;
      float bv = 0.f;
      for (int q = 0; q < G; ++q) {
        if ((taken[q >> 6] >> (q & 63)) & 1ull) continue;
        const float s = s_l[w][g * G + q];
        if (bi < 0 || s > bv) {
          bv = s;
          bi = q;
        }
      }
      taken[bi >> 6] |= 1ull << (bi & 63);
      const int e = g * G + bi;
      idx[(size_t)t * K + g * kp + j] = e;
      gate[(size_t)t * K + g * kp + j] = s_p[w][e];
    }
  }
}

hipError_t launch_route(const float* partial, int ksplit, int T, int N, int M, int kp,
                        const float* bias, float* logits_out, float* probs, int32_t* idx,
                        float* gate, hipStream_t st, int* zero, int n_zero) {
  if (ksplit < 1 || ksplit > kMaxRouterSplit || n_zero < 0 || (n_zero > 0 && !zero))
    return hipErrorInvalidValue;
  dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
  hipLaunchKernelGGL(k_route, grid, dim3(64 * kRouteWaves), 0, st, partial, ksplit, T, N, M, kp,
                     bias, logits_out, probs, idx, gate, zero, n_zero);
  return hipGetLastError();
}

}  // namespace moge
