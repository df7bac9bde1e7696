// Grouped SwiGLU expert FFN: the grouped matmul of the MoGE layer.
//
// The TechWalker page (section 三 推理性能优化, SwiftGMM) describes the grouped
// matmul as the largest share of decode latency and its best kernel as one that
// streams the expert weights near the weight-transfer bound, picking a GEMV-like
// or GEMM-like mode from the per-expert workload.  On MI355X the weight stream is
// the HBM stream; the contraction itself goes through MFMA in both regimes.
//
// Streaming kernels (this file): one wave owns 16 output features of one expert
// and the whole contraction; it streams those 16 weight rows exactly once per
// group of up to 64 of the expert's rows (A operand = weight rows, loaded with
// non-temporal 16-byte loads; B operand = the expert's activation rows, which
// stay in L2).  SwiGLU is applied to the float32 accumulators before the single
// rounding of H.
#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

struct SegView {
  int lo, cnt;
};

__device__ __forceinline__ SegView expert_rows(const FfnSeg& g, int e, int total_rows_cap) {
  SegView v;
  if (g.offsets) {
    int lo = g.offsets[e], hi = g.offsets[e + 1];
    lo = max(0, min(lo, total_rows_cap));
    hi = max(lo, min(hi, total_rows_cap));
    v.lo = lo;
    v.cnt = hi - lo;
  } else {
    v.lo = 0;
    v.cnt = g.rows;
  }
  return v;
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU, MS row-subtiles of 16 per pass over the weights
// ---------------------------------------------------------------------------
template <typename E, int MS>
__device__ __forceinline__ void gateup_pass(const FfnSeg& g, int d, int e, int n0, int lo,
                                            int cnt, int m0) {
  const int l = threadIdx.x & 63, ln = l & 15, kq = (l >> 4) * 8;
  const E* wg = static_cast<const E*>(g.w_gate) + ((size_t)e * g.inter + n0 + ln) * d + kq;
  const E* wu = static_cast<const E*>(g.w_up) + ((size_t)e * g.inter + n0 + ln) * d + kq;
  const E* xb[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int r = lo + min(m0 + ms * 16 + ln, cnt - 1);
    const int src = g.row_src ? g.row_src[r] / g.row_div : r;
    xb[ms] = static_cast<const E*>(g.x) + (size_t)src * d + kq;
  }
  f32x4 ag[MS], au[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    ag[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[ms] = ag[ms];
  }
#pragma unroll 4
  for (int k = 0; k < d; k += 32) {
    Frag8<E> fg, fu;
    fg.load_nt(wg + k);
    fu.load_nt(wu + k);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      Frag8<E> fx;
      fx.load(xb[ms] + k);
      ag[ms] = mfma_step(fg, fx, ag[ms]);
      au[ms] = mfma_step(fu, fx, au[ms]);
    }
  }
  // lane l holds features n0 + 4*(l/16) + i of row m0 + ms*16 + l%16
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int rr = m0 + ms * 16 + ln;
    if (rr < cnt) {
      f32x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = silu(ag[ms][i]) * au[ms][i];
      store4(static_cast<E*>(g.h) + (size_t)(lo + rr) * g.inter + n0 + 4 * (l >> 4), h);
    }
  }
}

template <typename E>
__global__ __launch_bounds__(64) void k_ffn_gateup(FfnSeg a, FfnSeg b, int d, int items_a,
                                                   int rows_cap_a, int rows_cap_b) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int nb = g.inter / 16;
  const int e = item / nb, n0 = (item - e * nb) * 16;
  const SegView v = expert_rows(g, e, second ? rows_cap_b : rows_cap_a);
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      gateup_pass<E, 4>(g, d, e, n0, v.lo, v.cnt, m0);
    else if (rem > 32)
      gateup_pass<E, 3>(g, d, e, n0, v.lo, v.cnt, m0);
    else if (rem > 16)
      gateup_pass<E, 2>(g, d, e, n0, v.lo, v.cnt, m0);
    else
      gateup_pass<E, 1>(g, d, e, n0, v.lo, v.cnt, m0);
  }
}

// ---------------------------------------------------------------------------
// down projection: y[r, n0..n0+15] = H[r,:] . W_down[e, n0..n0+15, :]
// ---------------------------------------------------------------------------
template <typename E, int MS>
__device__ __forceinline__ void down_pass(const FfnSeg& g, int d, int e, int n0, int lo, int cnt,
                                          int m0) {
  const int l = threadIdx.x & 63, ln = l & 15, kq = (l >> 4) * 8;
  const int I = g.inter;
  const E* wd = static_cast<const E*>(g.w_down) + ((size_t)e * d + n0 + ln) * I + kq;
  const E* hb[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
    hb[ms] = static_cast<const E*>(g.h) + (size_t)(lo + min(m0 + ms * 16 + ln, cnt - 1)) * I + kq;
  f32x4 acc[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < I; k += 32) {
    Frag8<E> fw;
    fw.load_nt(wd + k);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      Frag8<E> fh;
      fh.load(hb[ms] + k);
      acc[ms] = mfma_step(fw, fh, acc[ms]);
    }
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int rr = m0 + ms * 16 + ln;
    if (rr < cnt) store4(static_cast<E*>(g.y) + (size_t)(lo + rr) * d + n0 + 4 * (l >> 4), acc[ms]);
  }
}

template <typename E>
__global__ __launch_bounds__(64) void k_ffn_down(FfnSeg a, FfnSeg b, int d, int items_a,
                                                 int rows_cap_a, int rows_cap_b) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int nb = d / 16;
  const int e = item / nb, n0 = (item - e * nb) * 16;
  const SegView v = expert_rows(g, e, second ? rows_cap_b : rows_cap_a);
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      down_pass<E, 4>(g, d, e, n0, v.lo, v.cnt, m0);
    else if (rem > 32)
      down_pass<E, 3>(g, d, e, n0, v.lo, v.cnt, m0);
    else if (rem > 16)
      down_pass<E, 2>(g, d, e, n0, v.lo, v.cnt, m0);
    else
      down_pass<E, 1>(g, d, e, n0, v.lo, v.cnt, m0);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int seg_rows_cap(const FfnSeg& s) { return s.rows; }

hipError_t launch_ffn_gateup(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st) {
  const int items_a = a.n_exp * (a.inter / 16);
  const int items_b = b ? b->n_exp * (b->inter / 16) : 0;
  const FfnSeg bb = b ? *b : FfnSeg{};
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_gateup<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a,
                       seg_rows_cap(a), seg_rows_cap(bb));
  else
    hipLaunchKernelGGL(k_ffn_gateup<float>, grid, dim3(64), 0, st, a, bb, d, items_a,
                       seg_rows_cap(a), seg_rows_cap(bb));
  return hipGetLastError();
}

hipError_t launch_ffn_down(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st) {
  const int items_a = a.n_exp * (d / 16);
  const int items_b = b ? b->n_exp * (d / 16) : 0;
  const FfnSeg bb = b ? *b : FfnSeg{};
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_down<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a,
                       seg_rows_cap(a), seg_rows_cap(bb));
  else
    hipLaunchKernelGGL(k_ffn_down<float>, grid, dim3(64), 0, st, a, bb, d, items_a,
                       seg_rows_cap(a), seg_rows_cap(bb));
  return hipGetLastError();
}

}  // namespace moge
