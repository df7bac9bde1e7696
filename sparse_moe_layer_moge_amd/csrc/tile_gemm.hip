// MFMA tile path of the grouped expert FFN, for experts whose row count is above
// the streaming threshold (prefill batches; the shared experts of a large batch).
//
// The TechWalker page (section 三, SwiftGMM) has the grouped matmul switch between
// a GEMV-like and a GEMM-like mode by workload; this is the GEMM-like mode.  Each
// workgroup (4 waves, one per SIMD) computes one tile of 256 rows:
//   gate/up: 96 intermediate features (their 96 gate and 96 up weight rows), SwiGLU
//            in the epilogue, H rounded once;
//   down:    256 output columns.
// Every wave owns 128 rows x (96 | 128) weight rows, i.e. 8 row fragments x (6 | 8)
// weight fragments of 16x16 accumulators, which keeps the LDS bytes read per MFMA
// and the global bytes per flop low enough to feed the matrix cores.
//
// The contraction runs in stages of 32 through kStages LDS buffers.  Operands go
// from global memory straight into LDS (buffer loads with the LDS destination, one
// 16-row x 32-element MFMA fragment = 1 KiB per wave instruction, so LDS holds
// both operands in fragment order and every fragment read is 64 contiguous lanes
// of 16 bytes), issued kStages-1 stages ahead of their use; a stage boundary is a
// counted wait for the wave's own loads of that stage plus a workgroup barrier.
//
// The tiles of all experts form one list: for every expert above the threshold
// ceil(rows / 256) row tiles, each paired with every weight tile; the shared
// segment's tiles follow.  The list is built on the device from the expert
// offsets (no host synchronisation).  Consecutive list entries share the row tile
// and go to the same XCD, so an activation tile is read from one L2.
#include <limits.h>

#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "packed_layout.hpp"

namespace moge {

constexpr int kTileM = 256;        // rows per tile
constexpr int kTileK = 32;         // contraction elements per stage (one MFMA step)
constexpr int kStages = 4;         // LDS buffers; loads run kStages-1 stages ahead
constexpr int kTileThreads = 256;  // 4 waves: 2 (rows) x 2 (weight rows)
constexpr int kXcds = 8;
constexpr int kFragBytes = 1024;   // one bf16 fragment: 64 lanes x 16 bytes
constexpr int kAFrags = kTileM / 16;                   // 16 row fragments per stage
constexpr int kAStageBytes = kAFrags * kFragBytes;

// weight fragments per wave: gate/up 3 blocks x (gate, up); down 4 blocks of 32
// rows x 2 halves
template <bool GATEUP> struct TileShape {
  static constexpr int kWFrags = GATEUP ? 6 : 8;
  static constexpr int kWRows = 2 * kWFrags * 16;                  // weight rows per tile
  static constexpr int kBFrags = 2 * kWFrags;                      // per stage
  static constexpr int kBStageBytes = kBFrags * kFragBytes;
  static constexpr int kBlocksPerTile = GATEUP ? 6 : 8;            // packed blocks per tile
  static constexpr int kStageBytes = kAStageBytes + kBStageBytes;
  // loads per wave per stage: A fragments, B fragments
  static constexpr int kALoads = kAFrags / 4;
  static constexpr int kBLoads = kBFrags / 4;
  static constexpr int kLoads = kALoads + kBLoads;
};

typedef __attribute__((address_space(3))) void* LdsPtr;

// One wave instruction: 64 lanes x 16 bytes from a buffer straight into LDS at
// `dst` + 16 * lane (dst wave-uniform).  Written as inline asm so that the
// compiler does not treat every later LDS read as dependent on it (it would wait
// for all outstanding loads, draining the prefetch); the kernel counts these
// loads itself (wait_vmcnt) and orders LDS access with barriers.  The instruction
// takes its LDS address from M0, which nothing else in these kernels uses.
__device__ __forceinline__ void lds_dma16(Rsrc r, uint32_t voff, uint32_t soff, const void* dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(LdsPtr)dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// wait until at most N of this wave's vector-memory operations are outstanding
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Row tiles of expert e of a segment (0 if it takes the streaming path).
__device__ __forceinline__ int seg_expert_tiles(const TileSeg& g, int e, int* lo, int* cnt) {
  int l0, c;
  if (g.offsets) {
    l0 = g.offsets[e];
    int h = g.offsets[e + 1];
    l0 = max(0, min(l0, g.rows));
    h = max(l0, min(h, g.rows));
    c = h - l0;
  } else {
    l0 = 0;
    c = g.rows;
  }
  *lo = l0;
  *cnt = c;
  return c > g.thr ? (c + kTileM - 1) / kTileM : 0;
}

// Find the row tile `mt` of a segment: expert, first row, rows.  Every lane of the
// wave takes part (the prefix over experts is a wave scan).
__device__ __forceinline__ bool seg_find_tile(const TileSeg& g, int mt, int* e_out, int* row0,
                                              int* rows) {
  const int l = threadIdx.x & 63;
  int base = 0;
  for (int e0 = 0; e0 < g.n_exp; e0 += 64) {
    const int e = e0 + l;
    int lo = 0, cnt = 0;
    const int nt = e < g.n_exp ? seg_expert_tiles(g, e, &lo, &cnt) : 0;
    // inclusive prefix of nt across the wave
    int inc = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (l >= o) inc += v;
    }
    const int start = base + inc - nt;
    const bool mine = nt > 0 && mt >= start && mt < start + nt;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      const int e_hit = __shfl(e, src, 64);
      const int s_hit = __shfl(start, src, 64);
      const int lo_hit = __shfl(lo, src, 64);
      const int c_hit = __shfl(cnt, src, 64);
      const int j = mt - s_hit;
      *e_out = e_hit;
      *row0 = lo_hit + j * kTileM;
      *rows = min(kTileM, c_hit - j * kTileM);
      return true;
    }
    base += __shfl(inc, 63, 64);
  }
  return false;
}

__device__ __forceinline__ int seg_total_tiles(const TileSeg& g) {
  const int l = threadIdx.x & 63;
  int s = 0;
  for (int e = l; e < g.n_exp; e += 64) {
    int lo, cnt;
    s += seg_expert_tiles(g, e, &lo, &cnt);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  return s;
}

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads, 1) void k_ffn_tile(TileSeg a, TileSeg b, int d) {
  typedef bf16 E;
  typedef TileShape<GATEUP> S;
  __shared__ __attribute__((aligned(1024))) char lds[kStages][S::kStageBytes];
  __shared__ int s_tile[5];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  // ---- which tile ------------------------------------------------------------
  if (w == 0) {
    const int nta = GATEUP ? a.inter / (S::kWRows / 2) : d / S::kWRows;
    const int ntb = b.n_exp ? (GATEUP ? b.inter / (S::kWRows / 2) : d / S::kWRows) : 0;
    const int ma = seg_total_tiles(a);
    const int mb = b.n_exp ? seg_total_tiles(b) : 0;
    const int total = ma * nta + mb * ntb;
    const int chunk = (total + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
    const int t = x * chunk + i;
    int seg = -1, e = 0, row0 = 0, rows = 0, nt = 0;
    if (i < chunk && t < total) {
      bool found;
      if (t < ma * nta) {
        seg = 0;
        nt = t % nta;
        found = seg_find_tile(a, t / nta, &e, &row0, &rows);
      } else {
        seg = 1;
        const int u = t - ma * nta;
        nt = u % ntb;
        found = seg_find_tile(b, u / ntb, &e, &row0, &rows);
      }
      if (!found || rows <= 0) seg = -1;
    }
    if (l == 0) {
      s_tile[0] = seg;
      s_tile[1] = e;
      s_tile[2] = row0;
      s_tile[3] = rows;
      s_tile[4] = nt;
    }
  }
  __syncthreads();
  const int seg = s_tile[0];
  if (seg < 0) return;
  const TileSeg g = seg == 0 ? a : b;
  const int e = s_tile[1];
  const int row0 = s_tile[2], rows = s_tile[3];
  const int nt = s_tile[4];
  const int K = GATEUP ? d : g.inter;              // contraction length of this segment
  const int nk = K / kTileK;                       // stages = 32-steps

  // the wave index as a scalar: every load below has a wave-uniform destination
  const int wu = __builtin_amdgcn_readfirstlane(w);

  // ---- A: row fragments rb = 4*wave + i; lane l reads row 16*rb + l%16, elements
  // 8*(l/16) .. +7 of the stage (global: 16 rows x 64 contiguous bytes)
  const Rsrc xr = make_rsrc(g.x, (uint64_t)g.x_rows * K * sizeof(E));
  uint32_t a_voff[S::kALoads];
#pragma unroll
  for (int i = 0; i < S::kALoads; ++i) {
    const int r = (wu * S::kALoads + i) * 16 + (l & 15);
    const int rr = row0 + min(r, rows - 1);
    const int src = (GATEUP && g.row_src) ? g.row_src[rr] / g.row_div : rr;
    a_voff[i] = (uint32_t)(((size_t)src * K + (l >> 4) * 8) * sizeof(E));
  }
  // ---- B: stage fragment f = kBLoads*wave + i = (block f/2, half f%2)
  const uint32_t tb = kTileElems * sizeof(E);
  const bool packed = g.packed != nullptr;
  Rsrc br0, br1;
  if (GATEUP) {
    const size_t ee = (size_t)g.inter * d;
    br0 = packed ? make_rsrc(static_cast<const char*>(g.packed) + e * 2 * ee * sizeof(E), 2 * ee * sizeof(E))
                 : make_rsrc(static_cast<const E*>(g.w0) + e * ee, ee * sizeof(E));
    br1 = packed ? br0 : make_rsrc(static_cast<const E*>(g.w1) + e * ee, ee * sizeof(E));
  } else {
    const size_t ee = (size_t)d * g.inter;
    br0 = packed ? make_rsrc(static_cast<const char*>(g.packed) + e * ee * sizeof(E), ee * sizeof(E))
                 : make_rsrc(static_cast<const E*>(g.w0) + e * ee, ee * sizeof(E));
    br1 = br0;
  }
  uint32_t b_voff[S::kBLoads];   // per lane
  uint32_t b_soff[S::kBLoads];   // per wave: stage-0 offset of the fragment
  Rsrc b_rsrc[S::kBLoads];
#pragma unroll
  for (int i = 0; i < S::kBLoads; ++i) {
    const int f = wu * S::kBLoads + i;
    const int blk = f >> 1, half = f & 1;
    const int pb = nt * S::kBlocksPerTile + blk;
    if (packed) {
      b_voff[i] = l * 8 * sizeof(E);
      b_soff[i] = (uint32_t)(pb * nk * 2 + half) * tb;
      b_rsrc[i] = br0;
    } else {
      const int row = GATEUP ? pb * 16 + (l & 15) : pb * 32 + half * 16 + (l & 15);
      b_voff[i] = (uint32_t)(((size_t)row * K + (l >> 4) * 8) * sizeof(E));
      b_soff[i] = 0;
      b_rsrc[i] = (GATEUP && half) ? br1 : br0;
    }
  }
  // per stage: packed weights advance 2 tiles, row-major 32 elements
  const uint32_t b_step = packed ? 2 * tb : kTileK * sizeof(E);
  const uint32_t a_step = kTileK * sizeof(E);

  auto issue = [&](int kb) {
    char* st = lds[kb % kStages];
#pragma unroll
    for (int i = 0; i < S::kALoads; ++i)
      lds_dma16(xr, a_voff[i], kb * a_step, st + (wu * S::kALoads + i) * kFragBytes);
#pragma unroll
    for (int i = 0; i < S::kBLoads; ++i)
      lds_dma16(b_rsrc[i], b_voff[i], b_soff[i] + kb * b_step,
                      st + kAStageBytes + (wu * S::kBLoads + i) * kFragBytes);
  };

  // ---- wave tile: 128 rows x (kWFrags * 16) weight rows, as 32x32 MFMA blocks:
  // kTP = 4 row pairs (two 16-row fragments each) x kWP weight pairs.
  // v_mfma_f32_32x32x16_bf16: lane l supplies weight row l%32 and row l%32 of the
  // token block, 8 contraction elements each; with 16-row fragments in LDS, row
  // l%32 lives in fragment (l%32)/16 at lane (2h + l/32)*16 + l%16 for sub-step h
  // (h = 0, 1 covers the stage's 32 elements).  Both operands use the same element
  // assignment, so the products pair up whatever the hardware's k order.
  constexpr int kTP = 4, kWP = S::kWFrags / 2;
  const int wm = w & 1, wn = w >> 1;
  f32x16 acc[kWP][kTP];
#pragma unroll
  for (int q = 0; q < kWP; ++q)
#pragma unroll
    for (int p = 0; p < kTP; ++p)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][p][r] = 0.f;
  const int half32 = (l & 31) >> 4;   // which 16-row fragment of a 32-row block

  auto compute = [&](int kb) {
    const char* A = lds[kb % kStages];
    const char* B = A + kAStageBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lane_off = (((2 * h + (l >> 5)) * 16) + (l & 15)) * 16;
      bf16x8 wf[kWP], tf[kTP];
      // weight pair q: fragments (block wn*kWP + q, half 0 | 1)
#pragma unroll
      for (int q = 0; q < kWP; ++q)
        wf[q] = *reinterpret_cast<const bf16x8*>(B + ((wn * kWP + q) * 2 + half32) * kFragBytes + lane_off);
      // row pair p: fragments 8*wm + 2p + (0 | 1)
#pragma unroll
      for (int p = 0; p < kTP; ++p)
        tf[p] = *reinterpret_cast<const bf16x8*>(A + (wm * 8 + 2 * p + half32) * kFragBytes + lane_off);
#pragma unroll
      for (int p = 0; p < kTP; ++p)
#pragma unroll
        for (int q = 0; q < kWP; ++q)
          acc[q][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[q], tf[p], acc[q][p], 0, 0, 0);
    }
  };

  // prologue: stages 0 .. kStages-2 in flight
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < nk) issue(p);
  for (int kb = 0; kb < nk; ++kb) {
    // this wave's loads of stage kb are done when at most the loads of the later
    // stages already issued (up to kStages-2 of them) are outstanding
    const int later = min(kStages - 2, nk - 1 - kb);
    if (later >= 2)
      wait_vmcnt<2 * S::kLoads>();
    else if (later == 1)
      wait_vmcnt<S::kLoads>();
    else
      wait_vmcnt<0>();
    // every wave's loads of stage kb have landed, and every wave has finished
    // reading the buffer that stage kb + kStages - 1 now overwrites
    barrier_only();
    if (kb + kStages - 1 < nk) issue(kb + kStages - 1);
    compute(kb);
  }

  // ---- epilogue ----------------------------------------------------------------
  // acc[q][p]: lane l, register r holds weight row 8*(r/4) + 4*(l/32) + r%4 of pair
  // q for tile row 32*(4*wm + p) + l%32.  Gate/up pairs are (gate rows, up rows) of
  // 16 features: registers r < 8 are gate, r + 8 the up value of the same feature.
  E* out = static_cast<E*>(g.out);
#pragma unroll
  for (int p = 0; p < kTP; ++p) {
    const int r0 = wm * 128 + p * 32 + (l & 31);
    if (r0 >= rows) continue;
    const size_t orow = (size_t)(row0 + r0);
#pragma unroll
    for (int q = 0; q < kWP; ++q) {
      if (GATEUP) {
        const int fbase = (nt * S::kBlocksPerTile + wn * kWP + q) * 16 + 4 * (l >> 5);
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
          f32x4 hv;
#pragma unroll
          for (int k = 0; k < 4; ++k) hv[k] = silu(acc[q][p][gq * 4 + k]) * acc[q][p][gq * 4 + k + 8];
          store4(out + orow * g.inter + fbase + 8 * gq, hv);
        }
      } else {
        const int cbase = (nt * S::kBlocksPerTile + wn * kWP + q) * 32 + 4 * (l >> 5);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = acc[q][p][gq * 4 + k];
          store4(out + orow * d + cbase + 8 * gq, v);
        }
      }
    }
  }
}

bool tile_path_ok(int d, int inter) {
  return d % TileShape<false>::kWRows == 0 && d % kTileK == 0 && inter % kTileK == 0 &&
         inter % (TileShape<true>::kWRows / 2) == 0;
}

// Upper bound of a segment's row tiles, from host-known sizes only.
static long long tile_bound(const TileSeg& g) {
  if (g.n_exp == 0) return 0;
  if (!g.offsets) return g.rows > g.thr ? (g.rows + kTileM - 1) / kTileM : 0;
  const long long R = g.rows;
  const long long big = R / (g.thr + 1);                    // experts above the threshold
  return R / kTileM + (big < g.n_exp ? big : g.n_exp) + 1;
}

hipError_t launch_ffn_tile(bool gateup, int d, const TileSeg& a, const TileSeg* b, hipStream_t st) {
  const TileSeg bb = b ? *b : TileSeg{};
  const long long wa = gateup ? TileShape<true>::kWRows / 2 : TileShape<false>::kWRows;
  const long long nta = gateup ? a.inter / wa : d / wa;
  const long long ntb = b ? (gateup ? bb.inter / wa : d / wa) : 0;
  const long long bound = tile_bound(a) * nta + tile_bound(bb) * ntb;
  if (bound == 0) return hipSuccess;
  const long long grid = ((bound + kXcds - 1) / kXcds) * kXcds;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  if (gateup)
    hipLaunchKernelGGL(k_ffn_tile<true>, dim3((unsigned)grid), dim3(kTileThreads), 0, st, a, bb, d);
  else
    hipLaunchKernelGGL(k_ffn_tile<false>, dim3((unsigned)grid), dim3(kTileThreads), 0, st, a, bb, d);
  return hipGetLastError();
}

}  // namespace moge
