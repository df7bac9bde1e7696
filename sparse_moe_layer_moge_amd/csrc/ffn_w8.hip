// Weight-only int8 (W8A16) SwiGLU experts for decode batch sizes.
//
// Quantised deployment of the experts is part of the inference work the pages
// describe (TechWalker, section 三 推理性能优化: expert-aware quantisation; CSDN
// page: W8A8 loses under 1.2% accuracy).  This is its weight half: each expert
// weight row holds int8 codes q with one float32 scale s (weight = s * q), and
// the activations stay bf16.  At decode sizes the layer's time is the time to
// stream the expert weights from HBM; one byte per weight instead of two halves it.
//
// One wave owns 32 weight rows of one expert - the gate and up rows of 16
// intermediate features, or 32 rows of the down projection - and the whole
// contraction, as in the bf16 streaming kernels.  Per 64-element step a lane
// loads 16 codes of each of its two 16-row tiles with one 16-byte load, widens
// them to bf16 (exact: an int8 value has at most 8 significant bits) and feeds two
// 16x16x32 bf16 MFMAs with float32 accumulation.  The row scales multiply the
// float32 sums in the epilogue, before SwiGLU.  A wave loads the scales of all its
// row blocks once, before its weight stream starts, into LDS; the epilogue reads
// them from there, so it never waits on a vector load issued behind the weight
// ring (vector loads complete in order: such a wait would drain the ring).
#include <math.h>

#include "ffn_rows.hpp"
#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "w8_layout.hpp"

namespace moge {
namespace {

// Scales of a wave's row blocks: 32 per block (16 gate + 16 up rows, or 32 down
// rows), at most 8 blocks per wave (plan_blocks picks nblk <= 8).
constexpr int kW8MaxBlocks = 8;
constexpr int kW8ScalesPerBlock = 32;

// Copy the scales of blocks b0 .. b0+nblk-1 into lds[blk*32 + j]:
//   gate/up (s1 != nullptr): j < 16 -> s0[16*(b0+blk) + j], j >= 16 -> s1[16*(b0+blk) + j-16]
//   down    (s1 == nullptr): s0[32*(b0+blk) + j]
// One wave per workgroup: the barrier only orders its LDS writes before the reads.
__device__ __forceinline__ void stage_scales(float* lds, const float* s0, const float* s1, int b0,
                                             int nblk) {
  const int l = threadIdx.x & 63;
  for (int i = 4 * l; i < nblk * kW8ScalesPerBlock; i += 256) {
    const int blk = i / kW8ScalesPerBlock, j = i % kW8ScalesPerBlock;
    const float* src = s1 ? (j < 16 ? s0 + (b0 + blk) * 16 + j : s1 + (b0 + blk) * 16 + j - 16)
                          : s0 + (b0 + blk) * 32 + j;
    *reinterpret_cast<f32x4*>(lds + i) = *reinterpret_cast<const f32x4*>(src);
  }
  __syncthreads();
}

// two floats holding integers of at most 8 significant bits -> their bf16 pair
// (the low 16 bits of each are zero, so taking the high halves is exact)
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                               0x07060302u);
}

// 16 int8 codes (contraction elements 0..15 of a lane chunk) -> bf16 fragments of
// elements 0..7 (lo) and 8..15 (hi)
__device__ __forceinline__ void widen16(const u32x4& w, u32x4& lo, u32x4& hi) {
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = w[j];
    o[2 * j] = bf16_pair((float)(int8_t)(v & 0xffu), (float)(int8_t)((v >> 8) & 0xffu));
    o[2 * j + 1] = bf16_pair((float)(int8_t)((v >> 16) & 0xffu), (float)(int8_t)(v >> 24));
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// The weight stream of one wave over `ngrp` groups of BPS consecutive row blocks
// (two 16-row code tiles per block and step, so 2*BPS tiles per step, all against
// the same activation fragments) and MS 16-row subtiles of activations.  Lane l
// supplies, for both the codes and the activations, contraction elements
// 16*(l/16) + 0..7 of a step to the first MFMA and 16*(l/16) + 8..15 to the second,
// so each step's sum covers its 64 elements exactly once.  The loads run PW steps
// ahead of the MFMAs through a register ring that carries on across group
// boundaries; after a group's last step flush(g, acc) takes its sums (acc[2*sb+t]
// is tile t of block sb of the group).  Needs nsteps * ngrp >= PW.
template <int MS, int BPS, int PW, typename Flush>
__device__ __forceinline__ void stream_w8(Rsrc wr, uint32_t wv0, uint32_t blk_bytes, Rsrc xr,
                                          const uint32_t (&xv)[MS], int nsteps, int ngrp,
                                          Flush&& flush) {
  constexpr int NB = 2 * BPS;
  constexpr uint32_t kStepW = 2 * kW8TileBytes;  // both tiles of a block's step
  constexpr uint32_t kStepX = kW8Step * 2;       // 64 bf16 activations
  u32x4 wb[PW][NB];
  u32x4 xb[PW][MS][2];
  f32x4 acc[NB][MS];
  auto zero = [&]() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[nb][ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  int l_grp = 0, l_j = 0;
  auto load = [&](int slot) {
    const uint32_t wso = (uint32_t)l_grp * BPS * blk_bytes + (uint32_t)l_j * kStepW;
    const uint32_t xso = (uint32_t)l_j * kStepX;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      wb[slot][nb] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     wr, wv0 + (nb & 1) * kW8TileBytes, wso + (nb >> 1) * blk_bytes,
                     kLoadNonTemporal));
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      xb[slot][ms][0] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv[ms], xso, 0));
      xb[slot][ms][1] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv[ms] + 16, xso, 0));
    }
    if (++l_j == nsteps) {
      l_j = 0;
      ++l_grp;
    }
  };
  int c_grp = 0, c_cnt = 0;
  auto compute = [&](int slot) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x4 lo, hi;
      widen16(wb[slot][nb], lo, hi);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        acc[nb][ms] = mfma_bf16(lo, xb[slot][ms][0], acc[nb][ms]);
        acc[nb][ms] = mfma_bf16(hi, xb[slot][ms][1], acc[nb][ms]);
      }
    }
    if (++c_cnt == nsteps) {
      flush(c_grp, acc);
      zero();
      c_cnt = 0;
      ++c_grp;
    }
  };

  zero();
  const int total = nsteps * ngrp;
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

// Stream shape by row-subtile count: blocks per step and prefetch depth.  The
// activation fragments (32 bytes per lane, step and subtile) cost as many
// registers as a block's two code tiles, so with one subtile two blocks share them
// and the ring holds 4 steps of 4 KiB; every variant fits 3 waves per SIMD
// without spilling.
template <int MS> struct W8Shape { static constexpr int bps = 2, depth = 4; };
template <> struct W8Shape<2> { static constexpr int bps = 2, depth = 3; };
template <> struct W8Shape<3> { static constexpr int bps = 1, depth = 2; };
template <> struct W8Shape<4> { static constexpr int bps = 1, depth = 2; };

// ---------------------------------------------------------------------------
// gate/up + SwiGLU: H[r, f] = silu(s_g[f] * (x_r . q_g[f])) * (s_u[f] * (x_r . q_u[f]))
// for the features of `nblk` 16-feature blocks starting at block b0
// ---------------------------------------------------------------------------
template <int MS, int BPS, int PW>
__device__ __forceinline__ void gateup_pass_w8(const FfnSeg& g, int d, int e, int b0, int nblk,
                                               int lo, int cnt, int m0, float* lds) {
  const int l = threadIdx.x & 63, ln = l & 15, lq = l >> 4;
  const int I = g.inter;
  const int nsteps = d / kW8Step;
  const size_t ebytes = (size_t)2 * I * d;
  const Rsrc wr = make_rsrc(static_cast<const int8_t*>(g.p_gu) + e * ebytes, ebytes);
  const uint32_t wv0 = (uint32_t)(b0 * nsteps * 2) * kW8TileBytes + l * 16;
  const uint32_t blk_bytes = (uint32_t)nsteps * 2 * kW8TileBytes;
  const Rsrc xr = make_rsrc(g.x, (uint64_t)g.x_rows * d * 2);
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int r = lo + min(m0 + ms * 16 + ln, cnt - 1);
    const int src = g.row_src ? g.row_src[r] / g.row_div : r;
    xv[ms] = (uint32_t)(((size_t)src * d + 16 * lq) * 2);
  }
  bf16* const h = static_cast<bf16*>(g.h);
  stage_scales(lds, g.sc_gate + (size_t)e * I, g.sc_up + (size_t)e * I, b0, nblk);
  // lane l holds features 16*b + 4*(l/16) + i of row m0 + ms*16 + l%16
  stream_w8<MS, BPS, PW>(wr, wv0, blk_bytes, xr, xv, nsteps, nblk / BPS,
                         [&](int grp, const f32x4 (&acc)[2 * BPS][MS]) {
#pragma unroll
    for (int sb = 0; sb < BPS; ++sb) {
      const int blk = grp * BPS + sb, f0 = (b0 + blk) * 16;
      const float* sc = lds + blk * kW8ScalesPerBlock;
      const f32x4 cg = *reinterpret_cast<const f32x4*>(sc + 4 * lq);
      const f32x4 cu = *reinterpret_cast<const f32x4*>(sc + 16 + 4 * lq);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int rr = m0 + ms * 16 + ln;
        if (rr < cnt) {
          f32x4 hv;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            hv[i] = silu(acc[2 * sb][ms][i] * cg[i]) * (acc[2 * sb + 1][ms][i] * cu[i]);
          store4(h + (size_t)(lo + rr) * I + f0 + 4 * lq, hv);
        }
      }
    }
  });
}

template <int MS>
__device__ __forceinline__ void gateup_w8_depth(const FfnSeg& g, int d, int e, int b0,
                                                const SegView& v, int m0, float* lds) {
  constexpr int BPS = W8Shape<MS>::bps, PW = W8Shape<MS>::depth;
  const int nsteps = d / kW8Step;
  if (g.nblk % BPS == 0 && nsteps * (g.nblk / BPS) >= PW)
    gateup_pass_w8<MS, BPS, PW>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, lds);
  else
    gateup_pass_w8<MS, 1, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, lds);
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_gateup_w8(
    FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int per_expert = g.inter / 16 / g.nblk;
  const int e = item / per_expert, b0 = (item - e * per_expert) * g.nblk;
  const SegView v = expert_rows(g, e);
  __shared__ float lds[kW8MaxBlocks * kW8ScalesPerBlock];
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      gateup_w8_depth<4>(g, d, e, b0, v, m0, lds);
    else if (rem > 32)
      gateup_w8_depth<3>(g, d, e, b0, v, m0, lds);
    else if (rem > 16)
      gateup_w8_depth<2>(g, d, e, b0, v, m0, lds);
    else
      gateup_w8_depth<1>(g, d, e, b0, v, m0, lds);
  }
}

// ---------------------------------------------------------------------------
// down projection: y[r, c] = s_d[c] * (H[r,:] . q_d[c,:]) for the 32 columns c of
// each of `nblk` blocks starting at block b0
// ---------------------------------------------------------------------------
template <int MS, int BPS, int PW>
__device__ __forceinline__ void down_pass_w8(const FfnSeg& g, int d, int e, int b0, int nblk,
                                             int lo, int cnt, int m0, float* lds) {
  const int l = threadIdx.x & 63, ln = l & 15, lq = l >> 4;
  const int I = g.inter;
  const int nsteps = I / kW8Step;
  const size_t ebytes = (size_t)d * I;
  const Rsrc wr = make_rsrc(static_cast<const int8_t*>(g.p_down) + e * ebytes, ebytes);
  const uint32_t wv0 = (uint32_t)(b0 * nsteps * 2) * kW8TileBytes + l * 16;
  const uint32_t blk_bytes = (uint32_t)nsteps * 2 * kW8TileBytes;
  const Rsrc xr = make_rsrc(g.h, (uint64_t)g.rows * I * 2);
  uint32_t xv[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
    xv[ms] = (uint32_t)(((size_t)(lo + min(m0 + ms * 16 + ln, cnt - 1)) * I + 16 * lq) * 2);
  bf16* const y = static_cast<bf16*>(g.y);
  stage_scales(lds, g.sc_down + (size_t)e * d, nullptr, b0, nblk);
  stream_w8<MS, BPS, PW>(wr, wv0, blk_bytes, xr, xv, nsteps, nblk / BPS,
                         [&](int grp, const f32x4 (&acc)[2 * BPS][MS]) {
#pragma unroll
    for (int sb = 0; sb < BPS; ++sb) {
      const int blk = grp * BPS + sb, c0 = (b0 + blk) * 32;
      const float* sc = lds + blk * kW8ScalesPerBlock;
      const f32x4 c_lo = *reinterpret_cast<const f32x4*>(sc + 4 * lq);
      const f32x4 c_hi = *reinterpret_cast<const f32x4*>(sc + 16 + 4 * lq);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int rr = m0 + ms * 16 + ln;
        if (rr < cnt) {
          f32x4 a, b;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = acc[2 * sb][ms][i] * c_lo[i];
            b[i] = acc[2 * sb + 1][ms][i] * c_hi[i];
          }
          bf16* out = y + (size_t)(lo + rr) * d + c0 + 4 * lq;
          store4(out, a);
          store4(out + 16, b);
        }
      }
    }
  });
}

template <int MS>
__device__ __forceinline__ void down_w8_depth(const FfnSeg& g, int d, int e, int b0,
                                              const SegView& v, int m0, float* lds) {
  constexpr int BPS = W8Shape<MS>::bps, PW = W8Shape<MS>::depth;
  const int nsteps = g.inter / kW8Step;
  if (g.nblk % BPS == 0 && nsteps * (g.nblk / BPS) >= PW)
    down_pass_w8<MS, BPS, PW>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, lds);
  else
    down_pass_w8<MS, 1, 1>(g, d, e, b0, g.nblk, v.lo, v.cnt, m0, lds);
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void k_ffn_down_w8(
    FfnSeg a, FfnSeg b, int d, int items_a) {
  int item = blockIdx.x;
  const bool second = item >= items_a;
  const FfnSeg g = second ? b : a;
  if (second) item -= items_a;
  const int per_expert = d / 32 / g.nblk;
  const int e = item / per_expert, b0 = (item - e * per_expert) * g.nblk;
  const SegView v = expert_rows(g, e);
  __shared__ float lds[kW8MaxBlocks * kW8ScalesPerBlock];
  for (int m0 = 0; m0 < v.cnt; m0 += 64) {
    const int rem = v.cnt - m0;
    if (rem > 48)
      down_w8_depth<4>(g, d, e, b0, v, m0, lds);
    else if (rem > 32)
      down_w8_depth<3>(g, d, e, b0, v, m0, lds);
    else if (rem > 16)
      down_w8_depth<2>(g, d, e, b0, v, m0, lds);
    else
      down_w8_depth<1>(g, d, e, b0, v, m0, lds);
  }
}

// ---------------------------------------------------------------------------
// code tiles from int8 codes: one thread per 16-byte destination chunk
//   gate/up mode (src1 != nullptr): 16-row blocks, tile 0 from src0, tile 1 from src1
//   down mode: 32-row blocks, tile t = rows 32b + 16t .. 32b + 16t + 15
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_w8_pack(const int8_t* __restrict__ src0,
                                                 const int8_t* __restrict__ src1, int n_exp,
                                                 int rows, int K, int8_t* __restrict__ dst) {
  const int nsteps = K / kW8Step;
  const bool gu = src1 != nullptr;
  const int block_rows = gu ? 16 : 32;
  const int nblocks = rows / block_rows;
  const size_t total = (size_t)n_exp * (gu ? 2 * rows : rows) * K / 16;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c & 63);
    size_t tile = c >> 6;
    const int t = (int)(tile & 1);
    tile >>= 1;
    const int s = (int)(tile % nsteps);
    tile /= nsteps;
    const int b = (int)(tile % nblocks);
    const int e = (int)(tile / nblocks);
    const int8_t* src = (gu && t == 1) ? src1 : src0;
    const int row = b * block_rows + (gu ? 0 : 16 * t) + (lane & 15);
    const int k = s * kW8Step + (lane >> 4) * 16;
    *reinterpret_cast<u32x4*>(dst + c * 16) =
        *reinterpret_cast<const u32x4*>(src + ((size_t)e * rows + row) * K + k);
  }
}

// ---------------------------------------------------------------------------
// quantisation of bf16 weight rows: one wave per row.
//   s = max_k |w[k]| / 127 and q[k] = rint(w[k] / s) (ties to even), clamped to
//   [-127, 127], every step in float32; a row of zeros gets s = 0 and q = 0.
// The codes go straight to their places in the code tiles (layout as k_w8_pack).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xffff0000u);
}

__device__ __forceinline__ uint32_t code_byte(float w, float s) {
  const float q = s > 0.f ? fminf(fmaxf(rintf(w / s), -127.f), 127.f) : 0.f;
  return (uint32_t)((int)q) & 0xffu;
}

__global__ __launch_bounds__(256) void k_w8_quantize(const uint16_t* __restrict__ src0,
                                                     const uint16_t* __restrict__ src1, int n_exp,
                                                     int rows, int K, int8_t* __restrict__ dst,
                                                     float* __restrict__ sc0,
                                                     float* __restrict__ sc1) {
  const bool gu = src1 != nullptr;
  const int l = threadIdx.x & 63;
  const long long per_tensor = (long long)n_exp * rows;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (gu ? 2 : 1) * per_tensor) return;  // the whole wave leaves together
  const int t = (int)(w / per_tensor);
  const long long er = w - t * per_tensor;
  const int e = (int)(er / rows), r = (int)(er - (long long)e * rows);
  const uint16_t* row = (t ? src1 : src0) + er * K;

  float m = 0.f;
  for (int k = l * 8; k < K; k += 64 * 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[j])), fabsf(bf16_hi(v[j]))));
  }
  m = wave_max(m);
  const float s = m / 127.0f;
  if (l == 0) (t ? sc1 : sc0)[er] = s;

  const int nsteps = K / kW8Step;
  int b, rr, tt;
  int8_t* base;
  if (gu) {
    b = r / 16;
    tt = t;
    rr = r % 16;
    base = dst + (size_t)e * 2 * rows * K;
  } else {
    b = r / 32;
    tt = (r % 32) / 16;
    rr = r % 16;
    base = dst + (size_t)e * rows * K;
  }
  for (int c = l; c < K / 16; c += 64) {
    const int k0 = c * 16, step = k0 / kW8Step, q4 = (k0 % kW8Step) / 16;
    const size_t tile = ((size_t)b * nsteps + step) * 2 + tt;
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(row + k0);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(row + k0 + 8);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o[j] = code_byte(bf16_lo(v0[2 * j]), s) | code_byte(bf16_hi(v0[2 * j]), s) << 8 |
             code_byte(bf16_lo(v0[2 * j + 1]), s) << 16 | code_byte(bf16_hi(v0[2 * j + 1]), s) << 24;
      o[2 + j] = code_byte(bf16_lo(v1[2 * j]), s) | code_byte(bf16_hi(v1[2 * j]), s) << 8 |
                 code_byte(bf16_lo(v1[2 * j + 1]), s) << 16 |
                 code_byte(bf16_hi(v1[2 * j + 1]), s) << 24;
    }
    *reinterpret_cast<u32x4*>(base + tile * kW8TileBytes + (size_t)(rr + 16 * q4) * 16) = o;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_ffn_gateup_w8(int d, const FfnSeg& a0, const FfnSeg* b0, hipStream_t st) {
  FfnSeg a = a0, bb = b0 ? *b0 : FfnSeg{};
  // a block = 16 gate rows + 16 up rows of one byte per weight
  plan_blocks(a, b0 ? &bb : nullptr, 32.0 * d, 32.0 * d, a.inter / 16, b0 ? bb.inter / 16 : 0,
              2);
  const int items_a = a.n_exp * (a.inter / 16 / a.nblk);
  const int items_b = b0 ? bb.n_exp * (bb.inter / 16 / bb.nblk) : 0;
  if (items_a + items_b == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ffn_gateup_w8, dim3(items_a + items_b), dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

hipError_t launch_ffn_down_w8(int d, const FfnSeg& a0, const FfnSeg* b0, hipStream_t st) {
  FfnSeg a = a0, bb = b0 ? *b0 : FfnSeg{};
  // a block = 32 down rows over the segment's intermediate width
  plan_blocks(a, b0 ? &bb : nullptr, 32.0 * a.inter, b0 ? 32.0 * bb.inter : 0.0, d / 32,
              b0 ? d / 32 : 0, 2, kDownRounds);
  const int items_a = a.n_exp * (d / 32 / a.nblk);
  const int items_b = b0 ? bb.n_exp * (d / 32 / bb.nblk) : 0;
  if (items_a + items_b == 0) return hipSuccess;
  hipLaunchKernelGGL(k_ffn_down_w8, dim3(items_a + items_b), dim3(64), 0, st, a, bb, d, items_a);
  return hipGetLastError();
}

hipError_t launch_w8_pack(const int8_t* src0, const int8_t* src1, int n_exp, int rows, int K,
                          int8_t* dst, hipStream_t st) {
  const size_t chunks = (size_t)n_exp * (src1 ? 2 * rows : rows) * K / 16;
  if (chunks == 0) return hipSuccess;
  const size_t want = (chunks + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_w8_pack, dim3(blocks), dim3(256), 0, st, src0, src1, n_exp, rows, K, dst);
  return hipGetLastError();
}

hipError_t launch_w8_quantize(const void* src0, const void* src1, int n_exp, int rows, int K,
                              int8_t* dst, float* scale0, float* scale1, hipStream_t st) {
  const long long waves = (long long)(src1 ? 2 : 1) * n_exp * rows;
  if (waves == 0) return hipSuccess;
  const long long blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(k_w8_quantize, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(src0), static_cast<const uint16_t*>(src1), n_exp,
                     rows, K, dst, scale0, scale1);
  return hipGetLastError();
}

}  // namespace moge
