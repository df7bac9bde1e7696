// Grouped SwiGLU expert FFN: the grouped matmul of the MoGE layer.
//
// The TechWalker page (section 三 推理性能优化, SwiftGMM) describes the grouped
// matmul as the largest share of decode latency and its best kernel as one that
// streams the expert weights near the weight-transfer bound, choosing a GEMV-like
// or GEMM-like mode from the per-expert workload.  On MI355X the weight stream is
// the HBM stream; the contraction itself runs on MFMA in both regimes.
//
// Streaming kernels (this file): one wave owns 32 weight rows of one expert - the
// gate and up rows of 16 intermediate features, or 32 rows of the down
// projection - and the whole contraction.  It streams those rows once per group of
// up to 64 of the expert's token rows (stream_tile.hpp).  SwiGLU is applied to the
// float32 accumulators before the single rounding of H.
#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "packed_layout.hpp"
#include "stream_tile.hpp"

namespace moge {

struct SegView {
  int lo, cnt;
};

// rows of expert e; offsets from the caller are clamped into [0, rows]
__device__ __forceinline__ SegView expert_rows(const FfnSeg& g, int e) {
  SegView v;
  if (g.offsets) {
    int lo = g.offsets[e], hi = g.offsets[e + 1];
    lo = max(0, min(lo, g.rows));
    hi = max(lo, min(hi, g.rows));
    v.lo = lo;
    v.cnt = hi - lo;
  } else {
    v.lo = 0;
    v.cnt = g.rows;
  }
  return v;
}

// starting K step of an item (rotation; see stream_tile.hpp)
__device__ __forceinline__ int stagger(int item, int nsteps) { return (item * 5) % nsteps; }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: H[r, n0..n0+15] = silu(x_r . Wg[n]) * (x_r . Wu[n])
// ---------------------------------------------------------------------------
template <typename E, int MS, int PW>
__device__ __forceinline__ void gateup_pass(const FfnSeg& g, int d, int e, int n0, int lo,
                                            int cnt, int m0, int s0) {
  const int l = threadIdx.x & 63, ln = l & 15, kq = (l >> 4) * 8;
  const int nsteps = d / 32;
  const size_t expert_elems = (size_t)g.inter * d;
  const bool packed = g.p_gu != nullptr;
  // packed: the wave's gate and up tiles of a step are adjacent (packed_layout.hpp)
  const char* pbase = static_cast<const char*>(g.p_gu) + e * 2 * expert_elems * sizeof(E);
  const uint32_t tb = kTileElems * sizeof(E);
  const uint32_t po = (uint32_t)((n0 / 16) * nsteps * 2) * tb + l * 8 * sizeof(E);
  const uint32_t wo = (uint32_t)(((n0 + ln) * d + kq) * sizeof(E));
  const Rsrc wr[2] = {
      packed ? make_rsrc(pbase, 2 * expert_elems * sizeof(E))
             : make_rsrc(static_cast<const E*>(g.w_gate) + e * expert_elems, expert_elems * sizeof(E)),
      packed ? make_rsrc(pbase, 2 * expert_elems * sizeof(E))
             : make_rsrc(static_cast<const E*>(g.w_up) + e * expert_elems, expert_elems * sizeof(E))};
  const uint32_t wv[2] = {packed ? po : wo, packed ? po + tb : wo};
  const uint32_t wstep = packed ? 2 * tb : 32 * sizeof(E);
  const Rsrc xr = make_rsrc(g.x, (uint64_t)g.x_rows * d * sizeof(E));
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int r = lo + min(m0 + ms * 16 + ln, cnt - 1);
    const int src = g.row_src ? g.row_src[r] / g.row_div : r;
    xv[ms] = (uint32_t)(((size_t)src * d + kq) * sizeof(E));
  }
  f32x4 acc[2][MS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_tile<E, 2, MS, PW>(wr, wv, wstep, xr, xv, nsteps, s0, acc);
  // lane l holds features n0 + 4*(l/16) + i of row m0 + ms*16 + l%16
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int rr = m0 + ms * 16 + ln;
    if (rr < cnt) {
      f32x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = silu(acc[0][ms][i]) * acc[1][ms][i];
      store4(static_cast<E*>(g.h) + (size_t)(lo + rr) * g.inter + n0 + 4 * (l >> 4), h);
    }
  }
}

template <typename E, int MS>
__device__ __forceinline__ void gateup_dispatch_depth(const FfnSeg& g, int d, int e, int n0,
                                                      const SegView& v, int m0, int s0) {
  constexpr int PW = StreamDepth<E, MS>::value;
  if (d / 32 >= PW)
    gateup_pass<E, MS, PW>(g, d, e, n0, v.lo, v.cnt, m0, s0);
  else
    gateup_pass<E, MS, 1>(g, d, e, n0, v.lo, v.cnt, m0, s0);
}

template <typename E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_gateup(FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int nb = g.inter / 16;
  const int e = item / nb, n0 = (item - e * nb) * 16;
  const SegView v = expert_rows(g, e);
  const int s0 = stagger(item, d / 32);
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      gateup_dispatch_depth<E, 4>(g, d, e, n0, v, m0, s0);
    else if (rem > 32)
      gateup_dispatch_depth<E, 3>(g, d, e, n0, v, m0, s0);
    else if (rem > 16)
      gateup_dispatch_depth<E, 2>(g, d, e, n0, v, m0, s0);
    else
      gateup_dispatch_depth<E, 1>(g, d, e, n0, v, m0, s0);
  }
}

// ---------------------------------------------------------------------------
// down projection: y[r, n0..n0+31] = H[r,:] . W_down[e, n0..n0+31, :]
// ---------------------------------------------------------------------------
template <typename E, int MS, int PW>
__device__ __forceinline__ void down_pass(const FfnSeg& g, int d, int e, int n0, int lo, int cnt,
                                          int m0, int s0) {
  const int l = threadIdx.x & 63, ln = l & 15, kq = (l >> 4) * 8;
  const int I = g.inter;
  const int nsteps = I / 32;
  const size_t expert_elems = (size_t)d * I;
  const bool packed = g.p_down != nullptr;
  const uint32_t tb = kTileElems * sizeof(E);
  const Rsrc w = packed ? make_rsrc(static_cast<const char*>(g.p_down) + e * expert_elems * sizeof(E),
                                    expert_elems * sizeof(E))
                        : make_rsrc(static_cast<const E*>(g.w_down) + e * expert_elems,
                                    expert_elems * sizeof(E));
  const Rsrc wr[2] = {w, w};
  // packed: rows n0..n0+15 and n0+16..n0+31 of a step are adjacent tiles
  const uint32_t po = (uint32_t)((n0 / 32) * nsteps * 2) * tb + l * 8 * sizeof(E);
  const uint32_t wo = (uint32_t)(((n0 + ln) * I + kq) * sizeof(E));
  const uint32_t wv[2] = {packed ? po : wo,
                          packed ? po + tb : wo + (uint32_t)(16 * I * sizeof(E))};
  const uint32_t wstep = packed ? 2 * tb : 32 * sizeof(E);
  const Rsrc xr = make_rsrc(g.h, (uint64_t)g.rows * I * sizeof(E));
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
    xv[ms] = (uint32_t)(((size_t)(lo + min(m0 + ms * 16 + ln, cnt - 1)) * I + kq) * sizeof(E));
  f32x4 acc[2][MS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_tile<E, 2, MS, PW>(wr, wv, wstep, xr, xv, nsteps, s0, acc);
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int rr = m0 + ms * 16 + ln;
    if (rr < cnt) {
      E* out = static_cast<E*>(g.y) + (size_t)(lo + rr) * d + n0 + 4 * (l >> 4);
      store4(out, acc[0][ms]);
      store4(out + 16, acc[1][ms]);
    }
  }
}

template <typename E, int MS>
__device__ __forceinline__ void down_dispatch_depth(const FfnSeg& g, int d, int e, int n0,
                                                    const SegView& v, int m0, int s0) {
  constexpr int PW = StreamDepth<E, MS>::value;
  if (g.inter / 32 >= PW)
    down_pass<E, MS, PW>(g, d, e, n0, v.lo, v.cnt, m0, s0);
  else
    down_pass<E, MS, 1>(g, d, e, n0, v.lo, v.cnt, m0, s0);
}

template <typename E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_down(FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int nb = d / 32;
  const int e = item / nb, n0 = (item - e * nb) * 32;
  const SegView v = expert_rows(g, e);
  const int s0 = stagger(item, g.inter / 32);
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      down_dispatch_depth<E, 4>(g, d, e, n0, v, m0, s0);
    else if (rem > 32)
      down_dispatch_depth<E, 3>(g, d, e, n0, v, m0, s0);
    else if (rem > 16)
      down_dispatch_depth<E, 2>(g, d, e, n0, v, m0, s0);
    else
      down_dispatch_depth<E, 1>(g, d, e, n0, v, m0, s0);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_ffn_gateup(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st) {
  const int items_a = a.n_exp * (a.inter / 16);
  const int items_b = b ? b->n_exp * (b->inter / 16) : 0;
  const FfnSeg bb = b ? *b : FfnSeg{};
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_gateup<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a);
  else
    hipLaunchKernelGGL(k_ffn_gateup<float>, grid, dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

hipError_t launch_ffn_down(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st) {
  const int items_a = a.n_exp * (d / 32);
  const int items_b = b ? b->n_exp * (d / 32) : 0;
  const FfnSeg bb = b ? *b : FfnSeg{};
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_down<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a);
  else
    hipLaunchKernelGGL(k_ffn_down<float>, grid, dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

}  // namespace moge
