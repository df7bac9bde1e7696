// Weight-streaming MFMA tile: the inner loop of the decode-regime grouped GEMV.
//
// One wave accumulates acc[nb][ms] (16x16 float32 each) = W_nb[16 rows, K] x
// X_ms[16 rows, K]^T, where W_nb are NB blocks of 16 weight rows (the A operand,
// streamed from HBM with non-temporal buffer loads) and X_ms are MS blocks of 16
// activation rows (the B operand, L2-resident).  Every lane loads 8 contraction
// elements of every row block per K=32 step: a fixed per-lane byte offset (wv,
// xv) plus a wave-uniform step offset in a scalar register (j * wstep for the
// weights, j * 32 elements for the activations).  With row-major weights wstep is
// 32 elements and one load touches 16 rows; with the packed fragment layout a
// step's NB fragments are adjacent and a wave's whole weight stream is one
// contiguous range.
//
// The loads run PW steps ahead of the MFMAs through a register ring, so a wave
// keeps PW * NB KiB of weights in flight; that is what lets a few thousand waves
// cover the HBM latency.  `s0` rotates the starting step (the sum over K is the
// same in any order): waves that run at the same time then read different column
// offsets of their rows instead of all hitting the same offset together.
#pragma once

#include "moge_common.hpp"

namespace moge {

template <typename E, int NB, int MS, int PW>
__device__ __forceinline__ void stream_tile(const Rsrc (&wr)[NB], const uint32_t (&wv)[NB],
                                            uint32_t wstep, Rsrc xr, const uint32_t (&xv)[MS],
                                            int nsteps, int s0, f32x4 (&acc)[NB][MS]) {
  constexpr uint32_t kStepBytes = 32 * sizeof(E);
  Frag8<E> wb[PW][NB];
  Frag8<E> xb[PW][MS];
  auto load = [&](int slot, int s) {
    int j = s0 + s;
    j -= (j >= nsteps) ? nsteps : 0;
    const uint32_t so = (uint32_t)j * kStepBytes;
    const uint32_t wso = (uint32_t)j * wstep;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wb[slot][nb].template load_buf<kLoadNonTemporal>(wr[nb], wv[nb], wso);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) xb[slot][ms].template load_buf<0>(xr, xv[ms], so);
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = mfma_step(wb[slot][nb], xb[slot][ms], acc[nb][ms]);
  };

  // requires nsteps >= PW
#pragma unroll
  for (int p = 0; p < PW; ++p) load(p, p);
  int s = 0;
  for (; s + 2 * PW <= nsteps; s += PW) {
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      compute(p);
      load(p, s + p + PW);
    }
  }
  // slots hold steps s .. s+PW-1; nsteps - s is in [PW, 2*PW)
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    compute(p);
    if (s + PW + p < nsteps) load(p, s + PW + p);
  }
#pragma unroll
  for (int p = 0; p < PW; ++p)
    if (s + PW + p < nsteps) compute(p);
}

// stream_blocks: the same stream over `nblk` consecutive row blocks that share
// the activation rows (the next block's weights start blk_bytes further on; in
// the packed layout that is the very next byte).  The ring runs on across block
// boundaries, so a wave never drains its loads between blocks; after the last
// step of block b, flush(b, acc) consumes the block's sums and acc restarts at 0.
// Needs nblk * nsteps >= PW.
template <typename E, int NB, int MS, int PW, typename Flush>
__device__ __forceinline__ void stream_blocks(const Rsrc (&wr)[NB], const uint32_t (&wv)[NB],
                                              uint32_t wstep, uint32_t blk_bytes, Rsrc xr,
                                              const uint32_t (&xv)[MS], int nsteps, int nblk,
                                              int s0, Flush&& flush) {
  constexpr uint32_t kStepBytes = 32 * sizeof(E);
  Frag8<E> wb[PW][NB];
  Frag8<E> xb[PW][MS];
  f32x4 acc[NB][MS];
  auto zero = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // load side: block, rotated step index, steps done in the block (wave-uniform)
  int l_blk = 0, l_j = s0, l_cnt = 0;
  auto load = [&](int slot) {
    const uint32_t wso = (uint32_t)l_blk * blk_bytes + (uint32_t)l_j * wstep;
    const uint32_t xso = (uint32_t)l_j * kStepBytes;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wb[slot][nb].template load_buf<kLoadNonTemporal>(wr[nb], wv[nb], wso);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) xb[slot][ms].template load_buf<0>(xr, xv[ms], xso);
    l_j = (l_j + 1 == nsteps) ? 0 : l_j + 1;
    if (++l_cnt == nsteps) {
      l_cnt = 0;
      ++l_blk;
    }
  };
  // compute side
  int c_blk = 0, c_cnt = 0;
  auto compute = [&](int slot) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = mfma_step(wb[slot][nb], xb[slot][ms], acc[nb][ms]);
    if (++c_cnt == nsteps) {
      flush(c_blk, acc);
      zero();
      c_cnt = 0;
      ++c_blk;
    }
  };

  zero();
  const int total = nsteps * nblk;
#pragma unroll
  for (int p = 0; p < PW; ++p) load(p);
  int q = 0;
  for (; q + 2 * PW <= total; q += PW) {
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      compute(p);
      load(p);
    }
  }
  // slots hold steps q .. q+PW-1; total - q is in [PW, 2*PW)
#pragma unroll
  for (int p = 0; p < PW; ++p) {
    compute(p);
    if (q + PW + p < total) load(p);
  }
#pragma unroll
  for (int p = 0; p < PW; ++p)
    if (q + PW + p < total) compute(p);
}

// Prefetch depth by row-subtile count: deep for the decode case (MS = 1), less
// when the activation fragments and accumulators take more registers, so every
// bf16 variant fits 3 waves per SIMD; float fragments are twice as wide.
template <typename E, int MS> struct StreamDepth { static constexpr int value = 8; };
template <> struct StreamDepth<bf16, 2> { static constexpr int value = 5; };
template <> struct StreamDepth<bf16, 3> { static constexpr int value = 5; };
template <> struct StreamDepth<bf16, 4> { static constexpr int value = 4; };
template <> struct StreamDepth<float, 1> { static constexpr int value = 4; };
template <> struct StreamDepth<float, 2> { static constexpr int value = 2; };
template <> struct StreamDepth<float, 3> { static constexpr int value = 2; };
template <> struct StreamDepth<float, 4> { static constexpr int value = 1; };

// Depth of the paired stream (two row blocks per step sharing the activation
// fragments); 0 = no paired variant for this subtile count.
template <typename E, int MS> struct StreamPair { static constexpr int depth = 0; };
template <> struct StreamPair<bf16, 1> { static constexpr int depth = 5; };

}  // namespace moge
