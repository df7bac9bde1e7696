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
#include <atomic>

#include <math.h>

#include "moge_common.hpp"
#include "ffn_rows.hpp"
#include "moge_internal.hpp"
#include "packed_layout.hpp"
#include "stream_tile.hpp"

namespace moge {

// Every block accumulates its K steps in the same order (no rotation: measured,
// rotating the start step did not change the achieved bandwidth), so results do
// not depend on how blocks are grouped into waves.
constexpr int kStartStep = 0;

// Narrow segments get an even number of blocks per wave, so that the paired
// (two blocks per step) stream applies.
constexpr int kPairBlocks = 2;

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: H[r, f] = silu(x_r . Wg[f]) * (x_r . Wu[f]) for the features
// f of `nblk` consecutive 16-feature blocks starting at block b0
// ---------------------------------------------------------------------------
// BPS blocks per step: with BPS = 2 the wave streams two blocks side by side, so
// each activation fragment serves four weight tiles.
template <typename E, int MS, int PW, int BPS>
__device__ __forceinline__ void gateup_pass(const FfnSeg& g, int d, int e, int b0, int nblk,
                                            int lo, int cnt, int m0, int s0) {
  const int l = threadIdx.x & 63, ln = l & 15, kq = (l >> 4) * 8;
  const int nsteps = d / 32;
  const size_t expert_elems = (size_t)g.inter * d;
  const bool packed = g.p_gu != nullptr;
  // packed: a block's gate and up tiles of a step are adjacent, blocks follow
  // each other (packed_layout.hpp)
  const char* pbase = static_cast<const char*>(g.p_gu) + e * 2 * expert_elems * sizeof(E);
  const uint32_t tb = kTileElems * sizeof(E);
  const uint32_t po = (uint32_t)(b0 * nsteps * 2) * tb + l * 8 * sizeof(E);
  const uint32_t wo = (uint32_t)(((b0 * 16 + ln) * d + kq) * sizeof(E));
  const Rsrc rg = packed ? make_rsrc(pbase, 2 * expert_elems * sizeof(E))
                         : make_rsrc(static_cast<const E*>(g.w_gate) + e * expert_elems,
                                     expert_elems * sizeof(E));
  const Rsrc ru = packed ? make_rsrc(pbase, 2 * expert_elems * sizeof(E))
                         : make_rsrc(static_cast<const E*>(g.w_up) + e * expert_elems,
                                     expert_elems * sizeof(E));
  const uint32_t wstep = packed ? 2 * tb : 32 * sizeof(E);
  const uint32_t blk_bytes = packed ? nsteps * 2 * tb : 16 * d * sizeof(E);
  // tile 2*sb + t: gate (t = 0) or up (t = 1) rows of block sb of the group
  Rsrc wr[2 * BPS];
  uint32_t wv[2 * BPS];
#pragma unroll
  for (int sb = 0; sb < BPS; ++sb) {
    wr[2 * sb] = rg;
    wr[2 * sb + 1] = ru;
    wv[2 * sb] = (packed ? po : wo) + sb * blk_bytes;
    wv[2 * sb + 1] = (packed ? po + tb : wo) + sb * blk_bytes;
  }
  const Rsrc xr = make_rsrc(g.x, (uint64_t)g.x_rows * d * sizeof(E));
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int r = lo + min(m0 + ms * 16 + ln, cnt - 1);
    const int src = g.row_src ? g.row_src[r] / g.row_div : r;
    xv[ms] = (uint32_t)(((size_t)src * d + kq) * sizeof(E));
  }
  E* const h = static_cast<E*>(g.h);
  const int I = g.inter;
  // lane l holds features 16*b + 4*(l/16) + i of row m0 + ms*16 + l%16
  stream_blocks<E, 2 * BPS, MS, PW>(wr, wv, wstep, BPS * blk_bytes, xr, xv, nsteps, nblk / BPS,
                                     s0, [&](int grp, const f32x4 (&acc)[2 * BPS][MS]) {
#pragma unroll
    for (int sb = 0; sb < BPS; ++sb) {
      const int blk = grp * BPS + sb;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int rr = m0 + ms * 16 + ln;
        if (rr < cnt) {
          f32x4 hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = silu(acc[2 * sb][ms][i]) * acc[2 * sb + 1][ms][i];
          store4(h + (size_t)(lo + rr) * I + (b0 + blk) * 16 + 4 * (l >> 4), hv);
        }
      }
    }
  });
}

template <typename E, int MS>
__device__ __forceinline__ void gateup_dispatch_depth(const FfnSeg& g, int d, int e, int b0,
                                                      const SegView& v, int m0, int s0) {
  constexpr int PW = StreamDepth<E, MS>::value;
  constexpr int PW2 = StreamPair<E, MS>::depth;
  const int nsteps = d / 32;
  if (PW2 > 0 && g.nblk % 2 == 0 && nsteps * (g.nblk / 2) >= PW2)
    gateup_pass<E, MS, (PW2 > 0 ? PW2 : 1), 2>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
  else if (nsteps * g.nblk >= PW)
    gateup_pass<E, MS, PW, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
  else
    gateup_pass<E, MS, 1, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
}

template <typename E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_gateup(
    FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int per_expert = g.inter / 16 / g.nblk;
  const int e = item / per_expert, b0 = (item - e * per_expert) * g.nblk;
  const SegView v = expert_rows(g, e);
  const int s0 = kStartStep;
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      gateup_dispatch_depth<E, 4>(g, d, e, b0, v, m0, s0);
    else if (rem > 32)
      gateup_dispatch_depth<E, 3>(g, d, e, b0, v, m0, s0);
    else if (rem > 16)
      gateup_dispatch_depth<E, 2>(g, d, e, b0, v, m0, s0);
    else
      gateup_dispatch_depth<E, 1>(g, d, e, b0, v, m0, s0);
  }
}

// ---------------------------------------------------------------------------
// down projection: y[r, 32b .. 32b+31] = H[r,:] . W_down[e, 32b .. 32b+31, :]
// for `nblk` consecutive 32-row blocks starting at block b0
// ---------------------------------------------------------------------------
template <typename E, int MS, int PW, int BPS>
__device__ __forceinline__ void down_pass(const FfnSeg& g, int d, int e, int b0, int nblk, int lo,
                                          int cnt, int m0, int s0) {
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
  // packed: rows 32b..32b+15 and 32b+16..32b+31 of a step are adjacent tiles
  const uint32_t po = (uint32_t)(b0 * nsteps * 2) * tb + l * 8 * sizeof(E);
  const uint32_t wo = (uint32_t)(((b0 * 32 + ln) * I + kq) * sizeof(E));
  const uint32_t wstep = packed ? 2 * tb : 32 * sizeof(E);
  const uint32_t blk_bytes = packed ? nsteps * 2 * tb : 32 * I * sizeof(E);
  // tile 2*sb + t: rows 32*(b0+blk) + 16t .. +15 of block sb of the group
  Rsrc wr[2 * BPS];
  uint32_t wv[2 * BPS];
#pragma unroll
  for (int sb = 0; sb < BPS; ++sb) {
    wr[2 * sb] = w;
    wr[2 * sb + 1] = w;
    wv[2 * sb] = (packed ? po : wo) + sb * blk_bytes;
    wv[2 * sb + 1] = (packed ? po + tb : wo + (uint32_t)(16 * I * sizeof(E))) + sb * blk_bytes;
  }
  const Rsrc xr = make_rsrc(g.h, (uint64_t)g.rows * I * sizeof(E));
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
    xv[ms] = (uint32_t)(((size_t)(lo + min(m0 + ms * 16 + ln, cnt - 1)) * I + kq) * sizeof(E));
  E* const y = static_cast<E*>(g.y);
  stream_blocks<E, 2 * BPS, MS, PW>(wr, wv, wstep, BPS * blk_bytes, xr, xv, nsteps, nblk / BPS,
                                     s0, [&](int grp, const f32x4 (&acc)[2 * BPS][MS]) {
#pragma unroll
    for (int sb = 0; sb < BPS; ++sb) {
      const int blk = grp * BPS + sb;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int rr = m0 + ms * 16 + ln;
        if (rr < cnt) {
          E* out = y + (size_t)(lo + rr) * d + (b0 + blk) * 32 + 4 * (l >> 4);
          store4(out, acc[2 * sb][ms]);
          store4(out + 16, acc[2 * sb + 1][ms]);
        }
      }
    }
  });
}

template <typename E, int MS>
__device__ __forceinline__ void down_dispatch_depth(const FfnSeg& g, int d, int e, int b0,
                                                    const SegView& v, int m0, int s0) {
  constexpr int PW = StreamDepth<E, MS>::value;
  constexpr int PW2 = StreamPair<E, MS>::depth;
  const int nsteps = g.inter / 32;
  if (PW2 > 0 && g.nblk % 2 == 0 && nsteps * (g.nblk / 2) >= PW2)
    down_pass<E, MS, (PW2 > 0 ? PW2 : 1), 2>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
  else if (nsteps * g.nblk >= PW)
    down_pass<E, MS, PW, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
  else
    down_pass<E, MS, 1, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, s0);
}

template <typename E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_down(
    FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int per_expert = d / 32 / g.nblk;
  const int e = item / per_expert, b0 = (item - e * per_expert) * g.nblk;
  const SegView v = expert_rows(g, e);
  const int s0 = kStartStep;
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      down_dispatch_depth<E, 4>(g, d, e, b0, v, m0, s0);
    else if (rem > 32)
      down_dispatch_depth<E, 3>(g, d, e, b0, v, m0, s0);
    else if (rem > 16)
      down_dispatch_depth<E, 2>(g, d, e, b0, v, m0, s0);
    else
      down_dispatch_depth<E, 1>(g, d, e, b0, v, m0, s0);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Resident wave slots of the streaming kernels (3 waves per SIMD, 4 SIMDs per CU).
int device_cus() {
  // per-device cache; concurrent first calls store the same value
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static int stream_slots() { return 3 * 4 * device_cus(); }

// Blocks per wave for one segment: the divisor k <= 8 of its blocks per expert
// whose item size (k blocks) is closest to an even share of the launch's weight
// bytes over the planned rounds of resident waves.  Segments whose rows need more than one
// 16-row subtile run slower per byte, so they aim at half the share.
static int blocks_per_wave(int blocks_per_expert, double block_bytes, double share,
                           int multiple) {
  // a multiple of `multiple` when the expert's block count allows one
  if (blocks_per_expert % multiple) multiple = 1;
  int best = 1;
  double best_err = 1e300;
  for (int k = multiple; k <= 8; k += multiple) {
    if (blocks_per_expert % k) continue;
    const double err = fabs(k * block_bytes - share);
    if (err < best_err) {
      best_err = err;
      best = k;
    }
  }
  return best;
}

// rows that a segment's experts may hold: > 16 means more than one row subtile
static bool wide_rows(const FfnSeg& g) { return g.offsets == nullptr && g.rows > 16; }

void plan_blocks(FfnSeg& a, FfnSeg* b, double a_block, double b_block, int a_bpe, int b_bpe,
                 int multiple, double rounds) {
  const double total = a_block * a.n_exp * a_bpe + (b ? b_block * b->n_exp * b_bpe : 0.0);
  const double share = total / (stream_slots() * rounds);
  a.nblk = wide_rows(a) ? blocks_per_wave(a_bpe, a_block, share / 2, 1)
                        : blocks_per_wave(a_bpe, a_block, share, multiple);
  if (b)
    b->nblk = wide_rows(*b) ? blocks_per_wave(b_bpe, b_block, share / 2, 1)
                            : blocks_per_wave(b_bpe, b_block, share, multiple);
}

hipError_t launch_ffn_gateup(int dtype, int d, const FfnSeg& a0, const FfnSeg* b0, hipStream_t st) {
  const int es = dtype == 1 ? 2 : 4;
  FfnSeg a = a0, bb = b0 ? *b0 : FfnSeg{};
  // a block = 16 gate rows + 16 up rows over the whole contraction
  plan_blocks(a, b0 ? &bb : nullptr, 32.0 * d * es, 32.0 * d * es, a.inter / 16,
              b0 ? bb.inter / 16 : 0, kPairBlocks);
  const int items_a = a.n_exp * (a.inter / 16 / a.nblk);
  const int items_b = b0 ? bb.n_exp * (bb.inter / 16 / bb.nblk) : 0;
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_gateup<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a);
  else
    hipLaunchKernelGGL(k_ffn_gateup<float>, grid, dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

hipError_t launch_ffn_down(int dtype, int d, const FfnSeg& a0, const FfnSeg* b0, hipStream_t st) {
  const int es = dtype == 1 ? 2 : 4;
  FfnSeg a = a0, bb = b0 ? *b0 : FfnSeg{};
  // a block = 32 down rows over the segment's intermediate width
  plan_blocks(a, b0 ? &bb : nullptr, 32.0 * a.inter * es, b0 ? 32.0 * bb.inter * es : 0.0,
              d / 32, b0 ? d / 32 : 0, kPairBlocks, kDownRounds);
  const int items_a = a.n_exp * (d / 32 / a.nblk);
  const int items_b = b0 ? bb.n_exp * (d / 32 / bb.nblk) : 0;
  if (items_a + items_b == 0) return hipSuccess;
  dim3 grid(items_a + items_b);
  if (dtype == 1)
    hipLaunchKernelGGL(k_ffn_down<bf16>, grid, dim3(64), 0, st, a, bb, d, items_a);
  else
    hipLaunchKernelGGL(k_ffn_down<float>, grid, dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

}  // namespace moge
