// MFMA tile path of the grouped expert FFN, for experts whose row count is above
// the streaming threshold (mid-size decode batches, prefill batches, the shared
// experts of a large batch).
//
// The TechWalker page (section 三, SwiftGMM) has the grouped matmul switch between
// a GEMV-like and a GEMM-like mode by workload; these are the GEMM-like modes.  A
// workgroup computes one tile; there are two tile shapes, chosen per expert by its
// row count:
//   big   (above 128 rows): 256 rows x (192 gate/up features | 256 output columns);
//         gate/up: 8 waves (two per SIMD), 2 (rows) x 4 (weight rows), each 128
//         rows x 96 weight rows as 4 x 3 blocks of 32x32 float32 accumulators;
//         down: 8 waves, 2 x 4, each 128 rows x 64 columns as 4 x 2 blocks.  This
//         one is bound by the matrix cores.  The launches that split the
//         contraction or mix in 64-row tiles take a 96-feature gate/up tile on 4
//         waves (one per SIMD, 2 x 2, each again 128 x 96).
//   small (up to 128 rows): 64 rows x (64 gate/up features | 128 output columns);
//         4 waves, all on the same 64 rows, each with its own 32 weight rows.
//         Wide: 64 rows x (96 features, waves 2 (rows) x 2 (weight rows) | 256
//         columns, each wave 64 weight rows).  This one streams each expert's
//         weights once and is bound by HBM.
// gate/up applies SwiGLU in the epilogue and rounds H once.  The matrix
// instruction is v_mfma_f32_32x32x16_bf16.
//
// The contraction runs in stages of 64 elements through rings of LDS buffers,
// filled straight from global memory (buffer loads with the LDS destination).
// Every 16-lane quarter of such a wave instruction reads whole 128-byte lines:
//   A (activation rows): 8 rows x 128 bytes per instruction, each row's line stored
//     with its eight 16-byte chunks XOR-swizzled by the row index (chunk c of row r
//     at position c ^ ((r >> 1) & 7)), so the MFMA operand reads are free of bank
//     conflicts;
//   B (weight rows): in MFMA fragment order, one 16-row x 32-element fragment (1 KiB,
//     contiguous in the packed weight layout) per instruction.
// The loads of later stages are spread between the MFMAs of the current one; a
// stage boundary is a wait for the wave's own loads plus a workgroup barrier.  The
// big tile keeps 2 activation and 4 (gate/up) or 3 (down) weight stages in LDS
// (the 8-wave gate/up tile 2 of both, its stages being 32 + 48 KiB); the small
// tile keeps 6 of both (wide: 5 for gate/up, 4 for down), enough bytes in flight
// to cover HBM latency with one workgroup per CU (on int8 codes 4 of both, 3 for the wide down
// tile, two workgroups per CU).  An expert's last row tile is mostly partial: a
// wave whose 32-row blocks are not all filled runs the copy of the main loop for
// its count of filled blocks, which leaves out the MFMAs of the empty ones.
//
// The tiles of a segment form one list: for every expert in the shape's row range
// ceil(rows / tile rows) row tiles, each paired with every weight tile (and
// contraction slice), row tile fastest inside the expert's block (for 256-row
// tiles, inside groups of a few row tiles).  The list is
// built on the device from the expert offsets (no host synchronisation).  Each
// XCD takes a contiguous eighth of every segment's list, so neighbouring entries
// (an expert's row tiles of one weight tile, then its next weight tiles) run at
// the same time on one XCD and share its L2; the segment with the longer
// contraction is scheduled first.  A 256-row gate/up launch of many rounds runs
// persistent workgroups that keep their XCD's rounds together (k_ffn_tile).
#include <limits.h>

#include <type_traits>

#include "moge_common.hpp"
#include "moge_internal.hpp"
#include "packed_layout.hpp"
#include "w8_layout.hpp"

namespace moge {

constexpr int kTileK = 64;              // contraction elements per stage
constexpr int kLineBytes = kTileK * 2;  // one operand row of a stage (bf16)
constexpr int kTileThreads = 256;       // 4 waves (one per SIMD)
// Waves of a 256-row tile unless the launch says otherwise: 4 for gate/up, 8 (two
// per SIMD) for down.  With two waves per SIMD one wave's MFMAs run while the
// other waits; the down tiles gained about 1 % (T=4096: 0.660 -> 0.649 ms,
// T=16384: 2.425 -> 2.416 ms, same box).  A 96-feature gate/up tile on 8 waves of
// 64 x 96 read 43 % more from LDS per stage and lost 6 %; the 8-wave gate/up tile
// of the plain launches (TileShape::kXL) instead doubles the features, keeping
// each wave's 128 x 96: 29 % fewer operand bytes into LDS per flop (16384 tokens:
// gate/up 4.34 -> 4.07 ms, 4096 tokens: 1.215 -> 1.172 ms, same box).
template <bool GATEUP> constexpr int big_waves() { return GATEUP ? 4 : 8; }
// rounds of tiles per CU from which the 256-row tiles run persistent workgroups
constexpr int kPersistMinRounds = 24;
// polls of a round counter before a workgroup goes on regardless (each an L2 round
// trip and a short sleep; 16384 tokens, gate/up 4.05 ms with 16, 4.01 with 64,
// 3.99 with 256 polls)
constexpr int kRoundSpin = 256;
constexpr int kXcds = 8;
constexpr int kRowsPerLoad = 8;         // A rows one wave instruction moves
constexpr int kFragBytes = 1024;        // one 16 x 32 bf16 MFMA fragment
// The small shape on int8 codes: half-size weight stages, so two workgroups share
// a CU, each with 4-deep rings (one workgroup's tile changes, pipeline fills and
// epilogues overlap the other's loads; 2 x 4 and 3 x 3 measured alike, 1 x 6 slower)
constexpr int kSmallW8PerCU = 2;
constexpr int kSmallW8Depth = 4;

// W8: int8 weight codes (w8_layout.hpp) instead of bf16 weights, small shape only.
// WIDE: small tiles with 96 gate/up features (bf16) or 256 down columns instead of
// 64 and 128.  A launch with many tiles spreads the fixed per-tile cost (selection,
// pipeline fill, epilogue) over more bytes with fewer, wider tiles (T=456: bf16
// down 0.245 -> 0.218 ms and gate/up 0.381 -> 0.367 ms, int8 down 0.156 ->
// 0.144 ms); a launch of one round (the split shared segment of a small batch)
// keeps more, narrower tiles.
// WAVES: 0 for the shape's own wave count, 4 to force one wave per SIMD (a big
// tile in a launch whose other tiles run 4 waves), 8 for the big gate/up tile of
// 192 features on two waves per SIMD (kXL)
template <bool GATEUP, bool BIG, bool W8 = false, bool WIDE = false, int WAVES = 0> struct TileShape {
  // the big gate/up tile on 8 waves: 192 features (384 weight rows), each wave
  // 128 rows x 96 weight rows as the 4-wave tile's waves, two waves per SIMD
  static constexpr bool kXL = BIG && GATEUP && WAVES == 8;
  static constexpr int kM = BIG ? 256 : 64;                       // rows per tile
  static constexpr int kWRows =
      kXL ? 384 : (BIG || WIDE) ? (GATEUP ? 192 : 256) : 128;    // weight rows per tile
  static constexpr int kFeat = kWRows / 2;                         // gate/up features per tile
  static constexpr int kWaves = WAVES ? WAVES : (BIG ? big_waves<GATEUP>() : 4);
  static constexpr int kThreads = kWaves * 64;
  // waves along the rows
  static constexpr int kWavesM =
      BIG ? 2 : ((WIDE && GATEUP) ? 2 : 1);
  static constexpr int kWavesN = kWaves / kWavesM;
  static constexpr int kTP = kM / kWavesM / 32;                    // 32-row blocks per wave
  static constexpr int kBlocksPerTile = kWRows / 32;               // 32-row weight blocks
  static constexpr int kWP = kBlocksPerTile / kWavesN;             // ... per wave
  static constexpr int kPerCU = W8 ? kSmallW8PerCU : 1;            // workgroups per CU
  // stages in LDS (activations, weights).  The wide tiles' stages are bigger and
  // fit fewer deep (bf16 gate/up 32 KiB x 5, down 40 KiB x 4; int8 down 24 KiB x 3,
  // two workgroups per CU), about the bytes in flight of the narrow rings
  static constexpr int kSmallDepth =
      W8 ? (WIDE ? 3 : kSmallW8Depth) : (WIDE ? (GATEUP ? 5 : 4) : 6);
  // The 4-wave big gate/up tile's weight stages are smaller than its activation
  // stages (24 KiB against 32), so its weights run 3 stages ahead and fill the
  // LDS; the weights, not the activations, were the operand its MFMAs waited for.
  // The 8-wave one's stages (32 + 48 KiB) fit 2 deep
  static constexpr int kDA = BIG ? 2 : kSmallDepth;   // activation stages in LDS
  static constexpr int kDB = BIG ? (GATEUP ? (kXL ? 2 : 4) : 3) : kSmallDepth;   // weight stages in LDS
  static constexpr int kAStageBytes = kM * kLineBytes;
  // B stage: bf16 weights, kWRows / 8 fragments of 1 KiB; int8 codes, kWRows / 16
  // code tiles of 1 KiB (16 rows x 64 codes)
  static constexpr int kBStageBytes = kWRows * kTileK * (W8 ? 1 : 2);
  static constexpr int kLdsBytes = kDA * kAStageBytes + kDB * kBStageBytes;
  // wave instructions per stage: A (8 rows each), B (one fragment each)
  static constexpr int kALoads = kM / kRowsPerLoad / kWaves;
  static constexpr int kBLoads = kBStageBytes / kFragBytes / kWaves;
  // one load after every kEvery MFMAs (the 8-wave gate/up tile, whose next stage
  // has only the current one's MFMAs to arrive in, every second: 16384 tokens,
  // gate/up 4.12 -> 4.09 ms against every third, 4.28 every MFMA, 4.40 every fourth)
  static constexpr int kEvery = kXL ? 2 : BIG ? 3 : 1;
  static_assert(kALoads * kWaves * kRowsPerLoad == kM &&
                kBLoads * kWaves * kFragBytes == kBStageBytes, "loads cover a stage");
  static_assert(kDA <= kDB && (kDA == kDB || (kDA == 2 && kDB >= 3)), "ring depths");
  static_assert(kWP * kWavesN == kBlocksPerTile && kTP >= 1, "wave layout");
  static_assert(kLdsBytes * kPerCU <= 160 * 1024, "LDS budget");
  static_assert((kALoads + kBLoads) * kEvery <= 4 * kTP * kWP, "loads must fit in a stage");
  static_assert(!(W8 && BIG), "int8 codes use the small shape");
  static_assert(!WIDE || (!BIG && !(W8 && GATEUP)), "the wide tiles are small tiles");
};

// 8 int8 codes -> their bf16 values (exact: at most 8 significant bits)
__device__ __forceinline__ bf16x8 widen8(uint64_t c) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = (float)(int8_t)((c >> (16 * j)) & 0xffu);
    const float b = (float)(int8_t)((c >> (16 * j + 8)) & 0xffu);
    o[j] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                                 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}

// One wave instruction: 64 lanes x 16 bytes from a buffer straight into LDS at
// byte address `m0v` + 16 * lane (m0v wave-uniform).  Written as inline asm so that
// the compiler does not treat every later LDS read as dependent on it (it would wait
// for all outstanding loads, draining the prefetch); the kernel counts these loads
// itself (wait_vmcnt) and orders LDS access with barriers.  The instruction takes
// its LDS address from M0, which nothing else in these kernels uses; one wait state
// separates the M0 write from its use.
__device__ __forceinline__ void lds_dma16(Rsrc r, uint32_t voff, uint32_t soff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// the same, marked non-temporal (data read once)
__device__ __forceinline__ void lds_dma16_nt(Rsrc r, uint32_t voff, uint32_t soff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}
// wait until at most N of this wave's vector-memory operations are outstanding
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// the same for a wave-uniform n <= N
template <int N> __device__ __forceinline__ void wait_vmcnt_le(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N)
      wait_vmcnt<N>();
    else
      wait_vmcnt_le<N - 1>(n);
  }
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* LdsPtr;

// f(std::integral_constant<int, n>) for a wave-uniform 0 <= n <= N
template <int N, class F> __device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N)
      f(std::integral_constant<int, N>{});
    else
      with_count<N - 1>(n, f);
  }
}

// position of 16-byte chunk c of stage row r
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Row tiles of kM rows of expert e of a segment (0 unless its row count is in the
// range (thr, thr_hi] this tile shape serves).
template <int kM>
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
  return (c > g.thr && c <= g.thr_hi) ? (c + kM - 1) / kM : 0;
}

// Find the expert that owns row tile `mt` of a segment (row tiles numbered expert
// by expert): the expert, its first row and row count, the index of its first row
// tile and its number of row tiles.  Every lane of the wave takes part (the prefix
// over experts is a wave scan).
template <int kM>
__device__ __forceinline__ bool seg_find_expert(const TileSeg& g, int mt, int* e_out, int* lo_out,
                                                int* cnt_out, int* first_out, int* nrt_out) {
  const int l = threadIdx.x & 63;
  int base = 0;
  for (int e0 = 0; e0 < g.n_exp; e0 += 64) {
    const int e = e0 + l;
    int lo = 0, cnt = 0;
    const int nt = e < g.n_exp ? seg_expert_tiles<kM>(g, e, &lo, &cnt) : 0;
    // inclusive prefix of nt across the wave
    const int inc = wave_scan_add(nt);
    const int start = base + inc - nt;
    const bool mine = nt > 0 && mt >= start && mt < start + nt;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      *e_out = lane_value(e, src);
      *first_out = lane_value(start, src);
      *lo_out = lane_value(lo, src);
      *cnt_out = lane_value(cnt, src);
      *nrt_out = lane_value(nt, src);
      return true;
    }
    base += lane_value(inc, 63);
  }
  return false;
}

template <int kM> __device__ __forceinline__ int seg_total_tiles(const TileSeg& g) {
  const int l = threadIdx.x & 63;
  int s = 0;
  for (int e = l; e < g.n_exp; e += 64) {
    int lo, cnt;
    s += seg_expert_tiles<kM>(g, e, &lo, &cnt);
  }
  return lane_value(wave_scan_add(s), 63);
}

// A segment of at most 64 experts held across the lanes of a wave: lane e has
// expert e's row tiles, first row, rows and index of its first row tile.  Built
// once per workgroup (one round of loads for both segments), so that selecting
// a tile is a ballot over registers instead of another pass over the offsets.
struct SegLanes {
  int nt = 0, lo = 0, cnt = 0, start = 0;
};
template <int kM> __device__ __forceinline__ SegLanes seg_lanes(const TileSeg& g, int* total) {
  const int l = threadIdx.x & 63;
  SegLanes t;
  if (l < g.n_exp) t.nt = seg_expert_tiles<kM>(g, l, &t.lo, &t.cnt);
  const int inc = wave_scan_add(t.nt);
  t.start = inc - t.nt;
  *total = lane_value(inc, 63);
  return t;
}
// The expert that owns row tile `mt` (as seg_find_expert, from the lanes)
__device__ __forceinline__ bool seg_lanes_find(const SegLanes& t, int mt, int* e_out, int* lo_out,
                                               int* cnt_out, int* first_out, int* nrt_out) {
  const uint64_t m = __ballot(t.nt > 0 && mt >= t.start && mt < t.start + t.nt);
  if (!m) return false;
  const int src = __ffsll((long long)m) - 1;
  *e_out = src;
  *first_out = lane_value(t.start, src);
  *lo_out = lane_value(t.lo, src);
  *cnt_out = lane_value(t.cnt, src);
  *nrt_out = lane_value(t.nt, src);
  return true;
}

// The tile list of up to two segments on one tile shape (see the file comment).
// Every wave holds the totals (init); wave 0 picks the tile of list entry `it` of
// XCD `x` (select) and leaves its descriptor in `s_tile`: segment (-1: none),
// expert, first row, rows, weight tile, contraction slice.
template <bool GATEUP, bool BIG, bool W8, bool SPLIT, bool WIDE, int WAVES = 0>
struct TileList {
  typedef TileShape<GATEUP, BIG, W8, WIDE, WAVES> S;
  static constexpr bool kSliced = !BIG || SPLIT;   // this instantiation handles slices
  int nta = 0, ntb = 0, ma = 0, mb = 0, tot0 = 0, tot1 = 0, ch0 = 0, ch1 = 0;
  bool lanes = false, b_first = false;
  SegLanes la, lb;

  __device__ __forceinline__ void init(const TileSeg& a, const TileSeg& b, int d) {
    // entries per row tile: weight tiles times contraction slices (slice-major)
    nta = a.n_exp ? (GATEUP ? a.inter / S::kFeat : d / S::kWRows) * (kSliced ? a.ksplit : 1) : 0;
    ntb = b.n_exp ? (GATEUP ? b.inter / S::kFeat : d / S::kWRows) * (kSliced ? b.ksplit : 1) : 0;
    // segments of at most 64 experts: per-lane tables (one round of loads for
    // both); larger ones are scanned again for every tile
    lanes = a.n_exp <= 64 && b.n_exp <= 64;
    // row tiles of each segment, in locals: a choice at run time between two
    // members read back through the object would put the object in scratch memory
    int m0 = 0, m1 = 0;
    if (lanes) {
      if (a.n_exp) la = seg_lanes<S::kM>(a, &m0);
      if (b.n_exp) lb = seg_lanes<S::kM>(b, &m1);
    } else {
      m0 = a.n_exp ? seg_total_tiles<S::kM>(a) : 0;
      m1 = b.n_exp ? seg_total_tiles<S::kM>(b) : 0;
    }
    ma = m0;
    mb = m1;
    // every XCD takes an equal share of each segment; the segment with the longer
    // contraction (more work per tile) goes first, so its tiles do not pile up at
    // the end
    b_first = (GATEUP ? d : b.inter) > (GATEUP ? d : a.inter);
    const int w0 = m0 * nta, w1 = m1 * ntb;
    tot0 = b_first ? w1 : w0;
    tot1 = b_first ? w0 : w1;
    ch0 = (tot0 + kXcds - 1) / kXcds;
    ch1 = (tot1 + kXcds - 1) / kXcds;
  }
  // list entries of one XCD
  __device__ __forceinline__ int entries() const { return ch0 + ch1; }

  __device__ __forceinline__ void select(const TileSeg& a, const TileSeg& b, int it, int x,
                                         int* s_tile) const {
    const int l = threadIdx.x & 63;
    int seg = -1, e = 0, row0 = 0, rows = 0, nt = 0, ks = 0;
    int which = -1, t = 0;
    if (it < ch0) {
      t = x * ch0 + it;
      if (t < tot0) which = 0;
    } else {
      t = x * ch1 + (it - ch0);
      if (t < tot1) which = 1;
    }
    if (which >= 0) {
      seg = (which == 0) == b_first ? 1 : 0;
      const TileSeg& g = seg ? b : a;
      const int ntg = seg ? ntb : nta;
      const int ntc = ntg / (kSliced ? g.ksplit : 1);  // weight tiles per row tile
      // An expert with R row tiles owns entries [ntg * first, ntg * (first + R)),
      // row tile fastest: its R row tiles of one weight tile are neighbouring
      // entries, which run at the same time on the same XCD and share its L2.
      int lo = 0, cnt = 0, first = 0, nrt = 1;
      const bool found = lanes ? seg_lanes_find(seg ? lb : la, t / ntg, &e, &lo, &cnt, &first, &nrt)
                               : seg_find_expert<S::kM>(g, t / ntg, &e, &lo, &cnt, &first, &nrt);
      if (found) {
        const int j = t - ntg * first;
        int mt;
        if constexpr (BIG) {
          // an expert with many row tiles: groups of kGroupM row tiles, row tile
          // fastest inside a group, so that the workgroups running together on
          // an XCD share a few activation row tiles as well as a few weight
          // tiles (skewed batch of 16384 tokens: gate/up 4.69 -> 4.66 ms with
          // groups of 8, down 2.49 -> 2.44 ms with groups of 4).  An expert with
          // at most kGroupM row tiles keeps the plain order.
          // (the 8-wave gate/up tile: groups of 16; 16384 tokens, gate/up 4.09 ->
          // 4.07 ms against 8, 4.20 with 4)
          constexpr int kGroupM = GATEUP ? (S::kXL ? 16 : 8) : 4;
          const int span = kGroupM * ntg;
          const int grp = j / span, first_mt = grp * kGroupM;
          const int gs = min(nrt - first_mt, kGroupM);
          const int jj = j - grp * span;
          mt = first_mt + jj % gs;
          nt = jj / gs;
        } else {
          mt = j % nrt;
          nt = j / nrt;
        }
        ks = nt / ntc;
        nt -= ks * ntc;
        row0 = lo + mt * S::kM;
        rows = min(S::kM, cnt - mt * S::kM);
        if (rows <= 0) seg = -1;
      } else {
        seg = -1;
      }
    }
    if (l == 0) {
      s_tile[0] = seg;
      s_tile[1] = e;
      s_tile[2] = row0;
      s_tile[3] = rows;
      s_tile[4] = nt;
      s_tile[5] = ks;
    }
  }
};

// One tile: load, multiply and write it (every wave of the workgroup).
template <bool GATEUP, bool BIG, bool W8, bool SPLIT, bool WIDE, int WAVES = 0>
__device__ __forceinline__ void tile_compute(char* lds, const TileSeg& g, int d, int e, int row0,
                                             int rows, int nt, int kslice, int* arrive = nullptr) {
  typedef bf16 E;
  typedef TileShape<GATEUP, BIG, W8, WIDE, WAVES> S;
  constexpr bool kSliced = !BIG || SPLIT;
  char* const ldsA = lds;
  char* const ldsB = lds + S::kDA * S::kAStageBytes;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int K = GATEUP ? d : g.inter;              // contraction length of this segment
  const int nk = K / kTileK / (kSliced ? g.ksplit : 1);  // stages of this tile's slice
  const int kb0 = kslice * nk;                     // its first stage

  // LDS byte address of the buffers; the wave index as a scalar (every load below
  // has a wave-uniform destination)
  const uint32_t ldsA0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(LdsPtr)ldsA);
  const uint32_t ldsB0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(LdsPtr)ldsB);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // the lane's row within an 8-row load and the chunk it fetches for that row
  const int lr = l >> 3;

  // ---- A: stage rows 8 * (kALoads * wave + i) + l / 8
  const Rsrc xr = make_rsrc(g.x, (uint64_t)g.x_rows * K * sizeof(E));
  int a_src[S::kALoads];
#pragma unroll
  for (int i = 0; i < S::kALoads; ++i)
    a_src[i] = row0 + min((wu * S::kALoads + i) * kRowsPerLoad + lr, rows - 1);
  if (GATEUP && g.row_src) {
    // the source rows through the permutation: every load first, then one wait
    // (a wait per load puts several memory latencies into every tile's set-up)
    int pair[S::kALoads];
#pragma unroll
    for (int i = 0; i < S::kALoads; ++i) pair[i] = g.row_src[a_src[i]];
    const unsigned div = (unsigned)g.row_div;
#pragma unroll
    for (int i = 0; i < S::kALoads; ++i) a_src[i] = (int)((unsigned)pair[i] / div);
  }
  // Lanes of stage rows past the tile's last row take an offset past the end of
  // the activation buffer (under 4 GiB): the buffer's range check returns zeros
  // for them without a memory access, where a copy of the last row would cross
  // L2 and the load path for MFMA rows the epilogue drops.  Every load still goes
  // out, so the wait counts stay as they are.
  constexpr uint32_t kPastEnd = 0xFFFFFFF0u;
  uint32_t a_voff[S::kALoads];
#pragma unroll
  for (int i = 0; i < S::kALoads; ++i) {
    const int r = (wu * S::kALoads + i) * kRowsPerLoad + lr;
    a_voff[i] = r < rows ? (uint32_t)(((size_t)a_src[i] * K + kb0 * kTileK + swz_chunk(r, l & 7) * 8) *
                                      sizeof(E))
                         : kPastEnd;
  }
  // ---- B: the stage's weight rows in MFMA fragment order: fragment f = 2 rb + kh
  // holds rows 16 rb .. +15 and elements 32 kh .. +31 of the stage, lane j of the
  // fragment (16 bytes at 16 j) row j % 16, elements 8 (j / 16) .. +7.  This is the
  // packed weight layout's own tile format, so a packed fragment is one contiguous
  // 1 KiB read.  Row block rb is half rb % 2 of 32-row block rb / 2: for gate/up the
  // gate (half 0) or up rows of features kFeat nt + 16 (rb / 2) .. +15; for down,
  // output columns kWRows nt + 16 rb .. +15.
  const bool packed = W8 || g.packed != nullptr;
  Rsrc br0, br1;
  if (W8) {
    // int8 codes: gate/up part 2 * inter * d bytes per expert, down part d * inter
    const size_t eb = GATEUP ? (size_t)2 * g.inter * d : (size_t)d * g.inter;
    br0 = make_rsrc(static_cast<const char*>(g.packed) + e * eb, eb);
    br1 = br0;
  } else if (GATEUP) {
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
  const uint32_t tb = kTileElems * sizeof(E);      // one packed 16 x 32 tile
  uint32_t b_voff[S::kBLoads];
#pragma unroll
  for (int i = 0; i < S::kBLoads; ++i) {
    const int f = wu * S::kBLoads + i;
    const int rb = f >> 1, kh = f & 1;
    const int blk = rb >> 1, half = rb & 1;
    if (W8) {
      // code tiles of block pb: step j of 64 codes holds tiles 2j (half 0) and 2j + 1;
      // one stage is one step, so the wave's load i is code tile rb = f of the stage
      const int pb = nt * S::kBlocksPerTile + ((f >> 1));
      b_voff[i] = (uint32_t)(((pb * (K / kTileK) + kb0) * 2 + (f & 1)) * kW8TileBytes + l * 16);
    } else if (packed) {
      // packed block pb: step j of 32 elements holds tiles 2j (half 0), 2j + 1 (half 1);
      // a block has 2 * (K / 32) tiles, the slice starts at step 2 * kb0
      const int pb = nt * S::kBlocksPerTile + blk;
      b_voff[i] = (uint32_t)(((pb * (K / kTileK) + kb0) * 4 + kh * 2 + half) * tb + l * 16);
    } else {
      const int row = GATEUP ? nt * S::kFeat + blk * 16 + (l & 15) : nt * S::kWRows + rb * 16 + (l & 15);
      b_voff[i] = (uint32_t)(((size_t)row * K + kb0 * kTileK + kh * 32 + (l >> 4) * 8) * sizeof(E));
    }
  }
  // row-major gate/up: odd row blocks are up rows
  auto b_rsrc = [&](int i) {
    const int f = wu * S::kBLoads + i;
    return (GATEUP && ((f >> 1) & 1)) ? br1 : br0;
  };
  // per stage: packed weights advance 2 steps of (2 tiles), codes 1 step of 2 code
  // tiles, row-major weights 64 elements
  const uint32_t b_step = W8 ? 2 * kW8TileBytes : packed ? 4 * tb : kLineBytes;
  const uint32_t a_step = kLineBytes;

  // wave load i of the A rows of stage s, and of the B rows
  auto issue_a = [&](int i, int s) {
    const uint32_t st = ldsA0 + (uint32_t)((s % S::kDA) * S::kAStageBytes);
    lds_dma16(xr, a_voff[i], s * a_step, st + (wu * S::kALoads + i) * kRowsPerLoad * kLineBytes);
  };
  // non-temporal weight loads: bf16 64-row tiles of a segment that asks for them
  const bool b_nt = !BIG && !W8 && g.nt_weights;
  auto issue_b = [&](int i, int s) {
    const uint32_t st = ldsB0 + (uint32_t)((s % S::kDB) * S::kBStageBytes);
    if (b_nt)
      lds_dma16_nt(b_rsrc(i), b_voff[i], s * b_step, st + (wu * S::kBLoads + i) * kFragBytes);
    else
      lds_dma16(b_rsrc(i), b_voff[i], s * b_step, st + (wu * S::kBLoads + i) * kFragBytes);
  };

  // ---- wave tile: kTP 32-row blocks x kWP 32-weight-row blocks.
  // v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 of the weight block and
  // of the row block, contraction elements 8 (l / 32) .. +7 of the 16-element
  // sub-step; both operands use the same element assignment.
  constexpr int kTP = S::kTP, kWP = S::kWP;
  constexpr int kSub = kTileK / 16;                  // MFMA sub-steps per stage
  const int wm = w % S::kWavesM, wn = w / S::kWavesM;
  // 32-row blocks of this wave that hold rows of the tile.  The main loop has a
  // copy for every count, which leaves out the MFMAs of the empty blocks (their
  // loads still go out, in bounds, so that the wait counts stay the same): the
  // last, nearly empty row tile of an expert then costs little more than
  // streaming its weights once.  (A branch around each MFMA instead cost full
  // tiles 5-7 %, and made partial 256-row tiles slower than full ones.)
  const int nact = __builtin_amdgcn_readfirstlane(max(0, min(kTP, (rows - wm * kTP * 32 + 31) >> 5)));
  f32x16 acc[kWP][kTP];
#pragma unroll
  for (int q = 0; q < kWP; ++q)
#pragma unroll
    for (int p = 0; p < kTP; ++p)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][p][r] = 0.f;
  // a block's rows start at multiples of 32, so the swizzle depends on the lane only
  const int lane_row = (l & 31) * kLineBytes;
  const int lswz = ((l & 31) >> 1) & 7;

  // B fragment of sub-step h for lane l: row block 2 (32-row block) + (l % 32) / 16,
  // fragment h / 2, lane (2 (h % 2) + l / 32) * 16 + l % 16 of the fragment
  const int bhalf = ((l & 31) >> 4) * 2 * kFragBytes;
  auto read_frags = [&](const char* A, const char* B, int h, bf16x8 (&wf)[kWP], bf16x8 (&tf)[kTP]) {
    const int off = lane_row + (((2 * h + (l >> 5)) ^ lswz) << 4);
    const int boff = bhalf + (h >> 1) * kFragBytes + ((2 * (h & 1) + (l >> 5)) * 16 + (l & 15)) * 16;
#pragma unroll
    for (int q = 0; q < kWP; ++q) {
      if (W8) {
        // code tile 2 (32-row block) + (l % 32) / 16, chunk 16 h + l % 16 (row l % 16,
        // codes 16 h .. +15 of the stage), codes 8 (l / 32) .. +7 of the chunk
        const char* cp = B + (2 * (wn * kWP + q) + ((l & 31) >> 4)) * kW8TileBytes +
                         (h * 16 + (l & 15)) * 16 + 8 * (l >> 5);
        wf[q] = widen8(*reinterpret_cast<const uint64_t*>(cp));
      } else {
        wf[q] = *reinterpret_cast<const bf16x8*>(B + (wn * kWP + q) * 4 * kFragBytes + boff);
      }
    }
#pragma unroll
    for (int p = 0; p < kTP; ++p)
      tf[p] = *reinterpret_cast<const bf16x8*>(A + (wm * kTP + p) * 32 * kLineBytes + off);
  };

  // MFMAs of stage kb.  In between go out (one after every kEvery MFMAs, A first)
  // the A loads of stage kb + kDA - 1 when `next_a`, and the B loads of stage
  // kb + kDB - 1 when `next_b`.  Operand fragments are read one sub-step ahead.
  // Only the MFMAs of the wave's first `act` row blocks (a compile-time count).
  auto compute = [&](int kb, auto next_a, auto next_b, auto act) {
    constexpr int na = decltype(next_a)::value ? S::kALoads : 0;
    constexpr int nl = na + (decltype(next_b)::value ? S::kBLoads : 0);
    const char* A = ldsA + (kb % S::kDA) * S::kAStageBytes;
    const char* B = ldsB + (kb % S::kDB) * S::kBStageBytes;
    // the 8-wave gate/up tile reads each sub-step's fragments just before its
    // MFMAs (its registers hold no second set; the other wave on the SIMD runs
    // meanwhile)
    constexpr int kNB = S::kXL ? 1 : 2;
    bf16x8 wf[kNB][kWP], tf[kNB][kTP];
    if (kNB == 2) read_frags(A, B, 0, wf[0], tf[0]);
#pragma unroll
    for (int h = 0; h < kSub; ++h) {
      if (kNB == 1)
        read_frags(A, B, h, wf[0], tf[0]);
      else if (h + 1 < kSub)
        read_frags(A, B, h + 1, wf[(h + 1) % kNB], tf[(h + 1) % kNB]);
#pragma unroll
      for (int p = 0; p < kTP; ++p)
#pragma unroll
        for (int q = 0; q < kWP; ++q) {
          if (p < decltype(act)::value)
            acc[q][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[h % kNB][q], tf[h % kNB][p], acc[q][p], 0, 0, 0);
          const int m = (h * kTP + p) * kWP + q;
          const int j = m / S::kEvery;
          if (m % S::kEvery == S::kEvery - 1 && j < nl) {
            // keep the load where it is: the scheduler would otherwise bunch them
            __builtin_amdgcn_sched_barrier(0);
            if (j < na)
              issue_a(j, kb + S::kDA - 1);
            else
              issue_b(j - na, kb + S::kDB - 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
    }
  };

  // Loads complete in issue order as far as vmcnt is concerned.  Before the loop
  // go stages 0 .. kDB - 2 (A only up to kDA - 2), in stage order; the MFMAs of
  // stage j then issue A of stage j + kDA - 1, then B of stage j + kDB - 1.  At
  // the top of stage kb everything up to the last load stage kb needs has to be
  // in; what may still be outstanding is
  //   equal depths: the loads of stages kb+1 .. min(kb + kDA - 2, nk - 1);
  //   A depth 2, B deeper: the B loads issued after A of stage kb, i.e. those of
  //   stage kb + kDB - 2, if it exists (at kb = 0 this waits for a little more
  //   than it must: B of stages 1 .. kDB - 3 as well).
  auto pending = [&](int kb) {
    if (S::kDA == S::kDB) return (S::kALoads + S::kBLoads) * max(0, min(S::kDA - 2, nk - 1 - kb));
    return kb + S::kDB - 2 <= nk - 1 ? S::kBLoads : 0;
  };
  constexpr int kPendSteady = S::kDA == S::kDB ? (S::kDA - 2) * (S::kALoads + S::kBLoads) : S::kBLoads;

#pragma unroll
  for (int s = 0; s < S::kDB - 1; ++s) {
    if (s < nk) {
      if (s <= S::kDA - 2) {
#pragma unroll
        for (int i = 0; i < S::kALoads; ++i) issue_a(i, s);
      }
#pragma unroll
      for (int i = 0; i < S::kBLoads; ++i) issue_b(i, s);
    }
  }
  auto main_loop = [&](auto act) {
  int kb = 0;
  // both operands of a later stage go out
  for (; kb + S::kDB - 1 < nk; ++kb) {
    wait_vmcnt<kPendSteady>();
    // every wave's loads of stage kb are in, and every wave has finished reading
    // the buffers the loads issued during this stage overwrite (stage kb - 1's)
    barrier_only();
    compute(kb, std::true_type{}, std::true_type{}, act);
  }
  // only activations of a later stage go out
  for (; kb + S::kDA - 1 < nk; ++kb) {
    wait_vmcnt_le<kPendSteady>(pending(kb));
    barrier_only();
    compute(kb, std::true_type{}, std::false_type{}, act);
  }
  // nothing goes out
  for (; kb < nk; ++kb) {
    wait_vmcnt_le<kPendSteady>(pending(kb));
    barrier_only();
    compute(kb, std::false_type{}, std::false_type{}, act);
  }
  };
  with_count<kTP>(nact, main_loop);
  // the round counter learns of this tile once its operands are read; the
  // epilogue then runs while the rest of the round finishes
  if (arrive && threadIdx.x == 0)
    __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- epilogue ----------------------------------------------------------------
  // acc[q][p]: lane l, register r holds weight row 8*(r/4) + 4*(l/32) + r%4 of
  // block q for tile row 32*(kTP*wm + p) + l%32.  Gate/up blocks are (gate rows, up
  // rows) of 16 features: registers r < 8 are gate, r + 8 the up value of the same
  // feature.
  // The tile goes through LDS (the stage rings are free now), so that the global
  // stores are whole rows of 16-byte chunks instead of 8-byte pieces of 32 rows per
  // instruction.  An LDS row holds kNCp chunk slots (kNC used); chunk c of tile row
  // r sits at slot c ^ (r % kNCp), which keeps the scattered writes free of bank
  // conflicts.  Gate/up first applies SwiGLU in registers.
  constexpr int kOutCols = GATEUP ? S::kFeat : S::kWRows;   // output columns per tile
  if constexpr (W8) {
    // weight row scales: register group gq of block q is 4 consecutive rows
    // (gate/up: gate rows 4 gq .. of the block's 16 features, registers + 8 the up
    // rows of the same features; down: output columns)
#pragma unroll
    for (int q = 0; q < kWP; ++q) {
      const int blk = wn * kWP + q;
#pragma unroll
      for (int gq = 0; gq < (GATEUP ? 2 : 4); ++gq) {
        const int row = nt * kOutCols + blk * (GATEUP ? 16 : 32) + 8 * gq + 4 * (l >> 5);
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(g.sc0 + (size_t)e * (GATEUP ? g.inter : d) + row);
        f32x4 s1 = s0;
        if (GATEUP) s1 = *reinterpret_cast<const f32x4*>(g.sc1 + (size_t)e * g.inter + row);
#pragma unroll
        for (int p = 0; p < kTP; ++p)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[q][p][gq * 4 + k] *= s0[k];
            if (GATEUP) acc[q][p][gq * 4 + 8 + k] *= s1[k];
          }
      }
    }
  }
  if (SPLIT || (!BIG && g.ksplit > 1)) {
    // float32 partial sums straight from the accumulators: register group gq of
    // block q is 4 consecutive columns (down) or features (gate/up: registers
    // 4 gq .. +3 gate, 4 gq + 8 .. +11 up) of tile row 32 (kTP wm + p) + l % 32
    const int ld = GATEUP ? g.inter : d;
    const size_t plane = (size_t)g.rows * ld;
    float* const pg = g.part + kslice * plane;
    float* const pu = g.part + (size_t)g.ksplit * plane + kslice * plane;
#pragma unroll
    for (int p = 0; p < kTP; ++p) {
      const int r = (wm * kTP + p) * 32 + (l & 31);
      if (r < rows) {
#pragma unroll
        for (int q = 0; q < kWP; ++q) {
#pragma unroll
          for (int gq = 0; gq < (GATEUP ? 2 : 4); ++gq) {
            const int col = nt * kOutCols + (wn * kWP + q) * (GATEUP ? 16 : 32) + 8 * gq + 4 * (l >> 5);
            const size_t o = (size_t)(row0 + r) * ld + col;
            f32x4 v;
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = acc[q][p][gq * 4 + k];
            *reinterpret_cast<f32x4*>(pg + o) = v;
            if (GATEUP) {
#pragma unroll
              for (int k = 0; k < 4; ++k) v[k] = acc[q][p][gq * 4 + 8 + k];
              *reinterpret_cast<f32x4*>(pu + o) = v;
            }
          }
        }
      }
    }
  } else if constexpr (!SPLIT) {
  E* out = static_cast<E*>(g.out);
  constexpr int kNC = kOutCols * (int)sizeof(E) / 16;        // 16-byte chunks per row
  constexpr int kNCp = kNC <= 8 ? 8 : kNC <= 16 ? 16 : 32;   // ... rounded up to 2^k
  constexpr int kPitch = kNCp * 16;
  constexpr int kCPB = GATEUP ? 2 : 4;                       // chunks per 32-row block
  static_assert(kNC <= kNCp && S::kM * kPitch <= S::kLdsBytes, "the output tile fits in LDS");
  __syncthreads();   // every wave has finished reading the last stage
#pragma unroll
  for (int p = 0; p < kTP; ++p) {
    const int r = (wm * kTP + p) * 32 + (l & 31);
#pragma unroll
    for (int q = 0; q < kWP; ++q) {
#pragma unroll
      for (int gq = 0; gq < kCPB; ++gq) {
        f32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[k] = GATEUP ? silu(acc[q][p][gq * 4 + k]) * acc[q][p][gq * 4 + k + 8] : acc[q][p][gq * 4 + k];
        const int c = (wn * kWP + q) * kCPB + gq;
        store4(reinterpret_cast<E*>(lds + r * kPitch + ((c ^ (r & (kNCp - 1))) << 4) + 8 * (l >> 5)), v);
      }
    }
  }
  __syncthreads();
  const int ld = GATEUP ? g.inter : d;
  const int col0 = nt * kOutCols;
  for (int i = tid; i < rows * kNC; i += S::kThreads) {
    const int r = i / kNC, c = i - r * kNC;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kPitch + ((c ^ (r & (kNCp - 1))) << 4));
    // Outputs read back by a later launch, not by this one, go out non-temporal,
    // so that they do not push the launch's operands out of L2: the 256-row
    // tiles' H and y_perm (16384 tokens: layer 7.05 -> 7.00 ms, down 2.30 -> 2.27
    // ms) and the 64-row down tiles' y_perm (456 tokens: down 0.218 -> 0.204 ms).
    // The 64-row gate/up tiles keep H cached: their down launch reads it next
    // (non-temporal H cost that gate/up stage 1.4 %).
    if constexpr (BIG || !GATEUP)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (size_t)(row0 + r) * ld + col0 + c * 8));
    else
      *reinterpret_cast<u32x4*>(out + (size_t)(row0 + r) * ld + col0 + c * 8) = v;
  }
  }  // ksplit
}

// SPLIT (big shape only): every tile computes one slice of the contraction and
// writes float32 partial sums (a separate instantiation, so that the plain big
// kernels keep their registers).  The small shape handles both at run time.
// PERSIST (big shape): the workgroups (one per CU) walk their XCD's share of the
// list as the small shape's do, instead of one tile per workgroup.
template <bool GATEUP, bool BIG, bool W8, bool SPLIT = false, bool WIDE = false, bool PERSIST = false,
          int WV = 0>
__global__ __launch_bounds__(BIG ? (WV ? WV : big_waves<GATEUP>()) * 64 : kTileThreads, 1) void k_ffn_tile(TileSeg a, TileSeg b, int d) {
  typedef TileShape<GATEUP, BIG, W8, WIDE, WV> S;
  __shared__ __attribute__((aligned(1024))) char lds[S::kLdsBytes];
  // the tile descriptor lives in the last weight buffer, which the loads issued
  // before the main loop leave alone and later loads overwrite only after the
  // main loop's first barrier
  int* s_tile = reinterpret_cast<int*>(lds + S::kDA * S::kAStageBytes + (S::kDB - 1) * S::kBStageBytes);
  TileList<GATEUP, BIG, W8, SPLIT, WIDE, WV> list;
  list.init(a, b, d);
  // workgroup b runs on XCD b % 8 and takes that XCD's entry b / 8; the small shape
  // (launched with as many workgroups as fit the CUs) walks on to b / 8 + G, b / 8 + 2G,
  // ... (G workgroups per XCD), so the CUs of an XCD work on neighbouring entries
  const int x = blockIdx.x % kXcds;
  auto run_tile = [&](int it, int* arrive) {
    if ((threadIdx.x >> 6) == 0) list.select(a, b, it, x, s_tile);
    __syncthreads();
    const int seg = s_tile[0];
    if (seg >= 0)
      tile_compute<GATEUP, BIG, W8, SPLIT, WIDE, WV>(lds, seg == 0 ? a : b, d, s_tile[1], s_tile[2],
                                                 s_tile[3], s_tile[4],
                                                 decltype(list)::kSliced ? s_tile[5] : 0, arrive);
    else if (arrive && threadIdx.x == 0)
      __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if constexpr (BIG && !PERSIST) {
    // one tile per workgroup: the big shape's registers are nearly all taken by the
    // accumulators, and nothing may stay live across tiles
    if ((int)(blockIdx.x / kXcds) < list.entries()) run_tile(blockIdx.x / kXcds, nullptr);
  } else {
    const int gx = gridDim.x / kXcds;
    // Rounds (256-row tiles): the tiles of one round of an XCD's workgroups share a
    // few activation row tiles and weight tiles, which stay in the XCD's L2 only
    // while the tiles run side by side.  Left alone, the workgroups drift apart
    // over a launch of many rounds; so each one, after its tile's epilogue, waits
    // until every tile of its round has read its operands.  The wait is bounded
    // (only L2 reuse rides on it; a workgroup that never arrives costs about a
    // tile's time per round).  Skewed batch of 16384 tokens: L2 hit rate of the
    // gate/up launch 0.58 -> 0.76, reads beyond L2 20.8 -> 11.7 GB, layer 7.14 ->
    // 7.07 ms on one box.  A full barrier (waiting before the epilogue) gave the
    // same hit rate but no time; the 256-row down tiles lost time with rounds.
    int* const rounds = (BIG && PERSIST && a.rounds) ? a.rounds + 16 * x : nullptr;
    int round = 0;
    for (int it = blockIdx.x / kXcds; it < list.entries(); it += gx, ++round) {
      run_tile(it, rounds);
      // every wave is done with this tile's LDS (and the descriptor) before the next
      __syncthreads();
      if (rounds) {
        if (threadIdx.x == 0) {
          const int target = min(gx * (round + 1), list.entries());
          for (int i = 0; i < kRoundSpin &&
                          __hip_atomic_load(rounds, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target;
               ++i)
            __builtin_amdgcn_s_sleep(2);
        }
        __syncthreads();
      }
    }
  }
}


// Both projections of a decode batch of a few hundred tokens: the routed experts
// (a few dozen rows each) on 64-row tiles and the shared segment (every token) on
// 256-row tiles, in one launch per projection.  The shared tiles are bound by the
// matrix cores and the routed ones by HBM; side by side they keep both busy, where
// launches of their own leave the matrix cores idle during the routed one and
// HBM during the shared one.  A shared tile takes about as long as a few routed
// ones, so a fixed share of list entries per workgroup would leave the workgroups
// that drew one behind the rest: the workgroups of an XCD instead take the
// entries of that XCD's list (shared tiles first, or among the first) one at a
// time from a counter of their own, so neighbouring entries still run side by
// side there.  `sched` holds
// the 8 counters, 16 ints apart, zero at launch.  The shared tiles run 4 waves
// here, as the routed ones do.  The shared down tiles compute big.ksplit slices
// of the contraction (one or more) and write float32 partial sums to big.part:
// staging their 256 x 256 output through LDS as well took all 512 registers and
// spilled 96 more per lane.
template <bool GATEUP, bool WIDE>
__global__ __launch_bounds__(kTileThreads, 1) void k_ffn_mixed(TileSeg small, TileSeg big, int d,
                                                               int* sched) {
  constexpr bool BSPLIT = !GATEUP;
  typedef TileShape<GATEUP, false, false, WIDE> SS;
  typedef TileShape<GATEUP, true, false, false, 4> SB;
  static_assert(SS::kThreads == kTileThreads && SB::kThreads == kTileThreads,
                "both tile shapes run 4 waves");
  constexpr int kLds = SS::kLdsBytes > SB::kLdsBytes ? SS::kLdsBytes : SB::kLdsBytes;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  // each shape's descriptor in its own last weight buffer (see k_ffn_tile); the
  // entry a workgroup took beside the big shape's
  int* s_small = reinterpret_cast<int*>(lds + SS::kDA * SS::kAStageBytes + (SS::kDB - 1) * SS::kBStageBytes);
  int* s_big = reinterpret_cast<int*>(lds + SB::kDA * SB::kAStageBytes + (SB::kDB - 1) * SB::kBStageBytes);
  int* s_it = s_big + 8;
  constexpr int kOffS = SS::kDA * SS::kAStageBytes + (SS::kDB - 1) * SS::kBStageBytes;
  constexpr int kOffB = SB::kDA * SB::kAStageBytes + (SB::kDB - 1) * SB::kBStageBytes;
  static_assert(kOffS + 6 * 4 <= kOffB + 8 * 4 || kOffB + 9 * 4 <= kOffS,
                "the entry overlaps neither descriptor (6 ints each)");
  const TileSeg none{};
  TileList<GATEUP, false, false, false, WIDE> ls;
  ls.init(small, none, d);
  TileList<GATEUP, true, false, BSPLIT, false, 4> lb;
  lb.init(big, none, d);
  const int x = blockIdx.x % kXcds;
  const int nb = lb.entries(), ns = ls.entries(), n = nb + ns;
  // Gate/up: the shared entries go one in every k among the first nb * k entries
  // (k at most 4, and small enough that routed entries fill the gaps), so that
  // fewer CUs sit on the long shared tiles at once and more stream the routed
  // weights (456 tokens: gate/up 0.355 -> 0.351 ms).  Down: the shared entries
  // first (its sliced shared tiles are shorter; interleaving them made that
  // launch 0.5 % slower).
  constexpr int kMixEvery = GATEUP ? 4 : 1;
  const int k = nb > 0 ? min(kMixEvery, 1 + ns / nb) : 1;
  for (;;) {
    if (threadIdx.x == 0)
      *s_it = __hip_atomic_fetch_add(sched + 16 * x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = *s_it;
    if (it >= n) break;   // every workgroup reaches this: the counter only grows
    const bool is_big = it < nb * k && it % k == 0;
    const int ib = it / k;
    const int is = it < nb * k ? it - (it + k - 1) / k : it - nb;
    if ((threadIdx.x >> 6) == 0) {
      if (is_big)
        lb.select(big, none, ib, x, s_big);
      else
        ls.select(small, none, is, x, s_small);
    }
    __syncthreads();
    const int* t = is_big ? s_big : s_small;
    if (t[0] >= 0) {
      if (is_big)
        tile_compute<GATEUP, true, false, BSPLIT, false, 4>(lds, big, d, t[1], t[2], t[3], t[4],
                                                            BSPLIT ? t[5] : 0);
      else
        tile_compute<GATEUP, false, false, false, WIDE>(lds, small, d, t[1], t[2], t[3], t[4], t[5]);
    }
    // every wave is done with this tile's LDS (and the descriptors) before the next
    __syncthreads();
  }
}

int small_down_cols(bool wide) {
  return wide ? TileShape<false, false, false, true>::kWRows : TileShape<false, false>::kWRows;
}
int small_gateup_feats(bool wide) {
  return wide ? TileShape<true, false, false, true>::kFeat : TileShape<true, false>::kFeat;
}

bool tile_path_ok(int d, int inter) {
  // big tiles: 96-feature gate/up (split and mixed launches) and 256-column down
  // tiles; small tiles: 64 and 128 (implied); 64-element stages.  A width that is
  // a multiple of 64 and of 96 is one of 192, the 8-wave gate/up tile's features
  return d % TileShape<false, true>::kWRows == 0 && d % kTileK == 0 && inter % kTileK == 0 &&
         inter % TileShape<true, true>::kFeat == 0;
}

// Upper bound of a segment's row tiles of kM rows, from host-known sizes only.
static long long tile_bound(const TileSeg& g, int kM) {
  if (g.n_exp == 0) return 0;
  if (!g.offsets) return (g.rows > g.thr && g.rows <= g.thr_hi) ? (g.rows + kM - 1) / kM : 0;
  const long long R = g.rows;
  long long n_in = R / ((long long)g.thr + 1);              // experts above the threshold
  if (n_in > g.n_exp) n_in = g.n_exp;
  long long bound = R / kM + n_in + 1;
  if (g.thr_hi < INT_MAX) {                                 // each at most ceil(thr_hi / kM) tiles
    const long long b2 = n_in * ((g.thr_hi + kM - 1) / kM);
    if (b2 < bound) bound = b2;
  }
  return bound;
}

template <bool GATEUP, bool BIG, bool W8 = false, bool SPLIT = false, bool WIDE = false,
          bool PERSIST = false, int WV = 0>
static hipError_t launch_shape(int d, const TileSeg& a, const TileSeg* b, hipStream_t st) {
  typedef TileShape<GATEUP, BIG, W8, WIDE, WV> S;
  const TileSeg bb = b ? *b : TileSeg{};
  const long long wa = GATEUP ? S::kFeat : S::kWRows;
  const long long nta = (GATEUP ? a.inter / wa : d / wa) * ((!BIG || SPLIT) ? a.ksplit : 1);
  const long long ntb = b ? (GATEUP ? bb.inter / wa : d / wa) * ((!BIG || SPLIT) ? bb.ksplit : 1) : 0;
  // each segment's tiles are spread over the XCDs separately
  const long long ba = tile_bound(a, S::kM) * nta, bbn = tile_bound(bb, S::kM) * ntb;
  long long per_xcd = (ba + kXcds - 1) / kXcds + (bbn + kXcds - 1) / kXcds;
  if (per_xcd == 0) return hipSuccess;
  if (!BIG || PERSIST) {
    // as many workgroups as fit the CUs at once (the LDS rings take most of a CU's
    // LDS), each walking its XCD's share of the list: the bound counts every
    // expert that could fall in the range, and a launch that finds none stays cheap
    const long long slots = device_cus() * S::kPerCU / kXcds;
    if (per_xcd > slots) per_xcd = slots > 0 ? slots : 1;
  }
  const long long grid = per_xcd * kXcds;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_ffn_tile<GATEUP, BIG, W8, SPLIT, WIDE, PERSIST, WV>), dim3((unsigned)grid), dim3(S::kThreads),
                     0, st, a, bb, d);
  return hipGetLastError();
}

hipError_t launch_ffn_mixed(bool gateup, int d, const TileSeg& small, const TileSeg& big,
                            bool wide, int* sched, hipStream_t st) {
  // the shared down tiles: float32 partial sums of big.ksplit slices of whole
  // stages; the shared gate/up tiles: unsplit
  if (big.ksplit < 1 || big.ksplit > kMaxSlices || small.ksplit != 1 || !sched) return hipErrorInvalidValue;
  if (gateup ? big.ksplit != 1
             : big.n_exp && (!big.part || (big.inter / kTileK) % big.ksplit))
    return hipErrorInvalidValue;
  long long per_xcd;
  if (gateup) {
    typedef TileShape<true, true, false, false, 4> SB;
    const int fs = wide ? TileShape<true, false, false, true>::kFeat : TileShape<true, false>::kFeat;
    if (big.inter % SB::kFeat || small.inter % fs) return hipErrorInvalidValue;
    per_xcd = (tile_bound(big, SB::kM) * (big.inter / SB::kFeat) + kXcds - 1) / kXcds +
              (tile_bound(small, 64) * (small.inter / fs) + kXcds - 1) / kXcds;
  } else {
    typedef TileShape<false, true, false, false, 4> SB;
    const int cs = small_down_cols(wide);
    if (d % SB::kWRows || d % cs) return hipErrorInvalidValue;
    per_xcd = (tile_bound(big, SB::kM) * (d / SB::kWRows) * big.ksplit + kXcds - 1) / kXcds +
              (tile_bound(small, 64) * (d / cs) + kXcds - 1) / kXcds;
  }
  if (per_xcd == 0) return hipSuccess;
  const long long slots = device_cus() / kXcds;
  const long long grid = (per_xcd < slots ? per_xcd : (slots > 0 ? slots : 1)) * kXcds;
  const dim3 g((unsigned)grid), b(kTileThreads);
  if (gateup && wide)
    hipLaunchKernelGGL((k_ffn_mixed<true, true>), g, b, 0, st, small, big, d, sched);
  else if (gateup)
    hipLaunchKernelGGL((k_ffn_mixed<true, false>), g, b, 0, st, small, big, d, sched);
  else if (wide)
    hipLaunchKernelGGL((k_ffn_mixed<false, true>), g, b, 0, st, small, big, d, sched);
  else
    hipLaunchKernelGGL((k_ffn_mixed<false, false>), g, b, 0, st, small, big, d, sched);
  return hipGetLastError();
}

int tile_ksplit(int rows, int K, int col_tiles, int tile_rows) {
  constexpr int kPlanCUs = 256;   // MI355X; the split depends on the sizes only
  const int nk = K / kTileK;
  const long long tiles = (long long)((rows + tile_rows - 1) / tile_rows) * col_tiles;
  int best = 1;   // the most slices that still fit one round of workgroups
  for (int ks = 2; ks <= kMaxSlices; ++ks)
    if (nk % ks == 0 && nk / ks >= 12 && tiles * ks <= kPlanCUs) best = ks;
  return best;
}

hipError_t launch_ffn_tile(bool gateup, bool big, int d, const TileSeg& a, const TileSeg* b,
                           hipStream_t st, bool wide) {
  // big tiles with contraction slices: a launch of sliced segments only
  const bool sliced = a.ksplit > 1 || (b && b->ksplit > 1);
  if (big && sliced) {
    if ((a.n_exp && a.ksplit == 1) || (b && b->n_exp && b->ksplit == 1)) return hipErrorInvalidValue;
    return gateup ? launch_shape<true, true, false, true>(d, a, b, st)
                  : launch_shape<false, true, false, true>(d, a, b, st);
  }
  if (gateup && big) {
    // the 8-wave 192-feature tile: widths on the tile path are multiples of 64 and
    // of 96 (tile_path_ok), so of 192
    typedef TileShape<true, true, false, false, 8> S;
    if (a.inter % S::kFeat || (b && b->n_exp && b->inter % S::kFeat)) return hipErrorInvalidValue;
    // persistent workgroups in rounds for a launch of many rounds (counted in
    // 96-feature tiles)
    const long long tiles = 2 * (tile_bound(a, S::kM) * (a.inter / S::kFeat) +
                                 (b ? tile_bound(*b, S::kM) * (b->inter / S::kFeat) : 0));
    if (a.rounds && tiles >= (long long)kPersistMinRounds * device_cus())
      return launch_shape<true, true, false, false, false, true, 8>(d, a, b, st);
    return launch_shape<true, true, false, false, false, false, 8>(d, a, b, st);
  }
  if (gateup)
    return wide ? launch_shape<true, false, false, false, true>(d, a, b, st)
                : launch_shape<true, false>(d, a, b, st);
  if (big) {
    // Persistent 256-row down tiles for a launch of many rounds (16384 tokens:
    // 50 tiles per CU, down 2.46 -> 2.37 ms on one box); with few rounds (4096
    // tokens: 12 per CU) one tile per workgroup is faster (0.66 against 0.69 ms):
    // the hardware hands the next tile to whichever CU is free
    typedef TileShape<false, true> S;
    const long long tiles = tile_bound(a, S::kM) * (d / S::kWRows) +
                            (b ? tile_bound(*b, S::kM) * (d / S::kWRows) : 0);
    // (without rounds: with them the down tiles measured slower, 2.30 -> 2.39 ms)
    TileSeg a1 = a;
    a1.rounds = nullptr;
    if (tiles >= (long long)kPersistMinRounds * device_cus())
      return launch_shape<false, true, false, false, false, true>(d, a1, b, st);
    return launch_shape<false, true>(d, a1, b, st);
  }
  return wide ? launch_shape<false, false, false, false, true>(d, a, b, st)
              : launch_shape<false, false>(d, a, b, st);
}

bool tile_path_w8_ok(int d, int inter) {
  // 64-feature gate/up and 128-column down tiles of 64-code stages
  return d % TileShape<false, false, true>::kWRows == 0 && d % kW8Step == 0 &&
         inter % TileShape<true, false, true>::kFeat == 0 && inter % kW8Step == 0;
}

hipError_t launch_ffn_tile_w8(bool gateup, int d, const TileSeg& a, const TileSeg* b,
                              hipStream_t st, bool wide) {
  // int8 gate/up tiles stay narrow: the wide ones ran slower (T=456: 0.476 ->
  // 0.503 ms for the layer)
  if (gateup) return launch_shape<true, false, true>(d, a, b, st);
  return wide ? launch_shape<false, false, true, false, true>(d, a, b, st)
              : launch_shape<false, false, true>(d, a, b, st);
}

}  // namespace moge
