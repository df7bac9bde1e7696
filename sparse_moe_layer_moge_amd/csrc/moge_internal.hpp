// Internal launch interface of the MoGE library (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moge {

// ---- routing (router.hip) --------------------------------------------------
// partial[ks][t][e] = sum over the ks-th contraction split of x[t,:] . w_r[e,:]
hipError_t launch_router_scores(int dtype, const void* x, const void* w_router, int T, int d,
                                int N, int ksplit, float* partial, hipStream_t st);
// scores = sum_ks partial (+ bias); softmax over N; per-group top-K'.  The launch
// also zeroes n_zero ints at `zero` (the layer's expert work counters).
hipError_t launch_route(const float* partial, int ksplit, int T, int N, int M, int kp,
                        const float* bias, float* logits_out, float* probs, int32_t* idx,
                        float* gate, hipStream_t st, int* zero = nullptr, int n_zero = 0);
int router_ksplit(int dtype, int T, int d, int N);

// ---- permutation (permute.hip) ---------------------------------------------
constexpr int kPermTokens = 64;  // tokens per permutation block (one wave)
inline int perm_blocks(int T) { return (T + kPermTokens - 1) / kPermTokens; }
hipError_t launch_permute(const int32_t* idx, int T, int K, int N, int M, int32_t* blk_cnt,
                          int32_t* blk_base, int32_t* counts, int32_t* offsets,
                          int32_t* group_counts, int32_t* sorted_pair, int32_t* pair_row,
                          hipStream_t st);
// rows at or past *offsets_end (the device-side total row count) are left untouched
hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* sorted_pair,
                              const int32_t* offsets_end, int R, int K, int d, void* x_perm,
                              hipStream_t st);

// compute units of the current device (cached per device)
int device_cus();

// ---- expert FFN (ffn.hip) --------------------------------------------------
// One segment = a set of SwiGLU experts sharing a weight layout.  Row r of the
// segment reads activation row x[row_src ? row_src[r] / row_div : r].  Expert e
// owns rows offsets[e] .. offsets[e+1] (clamped into [0, rows]); offsets ==
// nullptr means a single expert owning rows [0, rows).  h and y hold `rows` rows.
struct FfnSeg {
  const void* x = nullptr;
  int x_rows = 0;                // rows of x (bounds of the activation buffer)
  const int32_t* row_src = nullptr;
  int row_div = 1;
  const int32_t* offsets = nullptr;
  int rows = 0;
  int n_exp = 0;
  int inter = 0;
  const void* w_gate = nullptr;  // [n_exp, inter, d]  row-major weights, or
  const void* w_up = nullptr;    // [n_exp, inter, d]
  const void* w_down = nullptr;  // [n_exp, d, inter]
  const void* p_gu = nullptr;    // packed gate/up parts, expert-strided (packed_layout.hpp)
  const void* p_down = nullptr;  // packed down parts, expert-strided
  const float* sc_gate = nullptr;  // int8 experts: per-channel scales of the gate rows
  const float* sc_up = nullptr;    //   [n_exp, inter], of the up rows [n_exp, inter]
  const float* sc_down = nullptr;  //   and of the down rows [n_exp, d] (w8_layout.hpp)
  int nblk = 1;                  // row blocks per wave (set by the launcher)
  int thr = 0x7fffffff;          // experts with more rows than this are left to the tile path
  void* h = nullptr;             // [rows, inter] dtype (gate/up output, down input)
  void* y = nullptr;             // [rows, d] dtype
};
// gate/up + SwiGLU for up to two segments in one launch (routed + shared)
hipError_t launch_ffn_gateup(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st);
// down projection for up to two segments in one launch
hipError_t launch_ffn_down(int dtype, int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st);
// Row blocks per wave (a.nblk, b->nblk) for a streaming launch: *_block = weight
// bytes of one row block, *_bpe = row blocks per expert; a segment of experts
// with at most 16 rows gets a multiple of `multiple` blocks where the block count
// per expert allows it.  The work items aim at `rounds` rounds of resident waves.
void plan_blocks(FfnSeg& a, FfnSeg* b, double a_block, double b_block, int a_bpe, int b_bpe,
                 int multiple = 1, double rounds = 1.0);
// Rounds of resident waves the down projection's work items aim at: its items
// are short (the contraction is the intermediate width), and more of them finish
// the launch sooner (a 64-token decode batch: 0.158 -> 0.157 ms for the stage in
// bf16, 0.093 -> 0.088 ms on int8 codes).
constexpr double kDownRounds = 2.0;

// ---- weight-only int8 expert FFN (ffn_w8.hip, bf16 activations) ------------
// Same segments, with p_gu / p_down holding int8 codes (w8_layout.hpp) and the
// sc_* scales set; every expert streams, whatever its row count.  Needs d, inter
// multiples of 64.
hipError_t launch_ffn_gateup_w8(int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st);
hipError_t launch_ffn_down_w8(int d, const FfnSeg& a, const FfnSeg* b, hipStream_t st);
// int8 codes [n_exp, rows, K] (gate/up pair when src1 != nullptr) -> code tiles
hipError_t launch_w8_pack(const int8_t* src0, const int8_t* src1, int n_exp, int rows, int K,
                          int8_t* dst, hipStream_t st);
// bf16 weights [n_exp, rows, K] (gate/up pair when src1 != nullptr) -> code tiles
// and per-row scales (scale0 for src0's rows, scale1 for src1's)
hipError_t launch_w8_quantize(const void* src0, const void* src1, int n_exp, int rows, int K,
                              int8_t* dst, float* scale0, float* scale1, hipStream_t st);

// ---- expert FFN, MFMA tile path (tile_gemm.hip, bf16) ----------------------
// By default routed experts with at most kStreamMaxRows rows take the streaming
// kernels; those with more take 64-row MFMA tiles up to kSmallTileMaxRows rows and
// 256-row tiles beyond (the layer moves these limits by the mean rows per expert).
// The shared experts (one segment of T rows) stream up to kSharedStreamMaxRows and
// take 64-row tiles up to kSharedSmallGateUpRows (gate/up) or kSharedSmallDownRows
// (down) and 256-row tiles beyond; a single segment too small to give one tile per
// CU has its contraction split over several tiles (tile_ksplit), so that it does
// not re-read its weights once per 64 rows.  A streamed segment of more than 32
// rows keeps three or four row subtiles of activations in registers and so few
// weight steps in flight; the 64-row tiles stage both operands in LDS instead.
// The limits are measured choices on MI355X.
constexpr int kStreamMaxRows = 32;
constexpr int kSharedStreamMaxRows = 32;
constexpr int kSmallTileMaxRows = 128;
constexpr int kSharedSmallGateUpRows = 128;
constexpr int kSharedSmallDownRows = 128;
struct TileSeg {
  const void* x = nullptr;         // activation rows (x, or H for the down projection)
  int x_rows = 0;
  const int32_t* row_src = nullptr;
  int row_div = 1;
  const int32_t* offsets = nullptr;  // nullptr: one expert with `rows` rows
  int rows = 0;
  int n_exp = 0;
  int inter = 0;
  int thr = 0;                     // the launch covers experts with more rows than
  int thr_hi = 0x7fffffff;         // thr and at most thr_hi
  const void* w0 = nullptr;        // row-major: gate (gate/up) or down
  const void* w1 = nullptr;        // row-major: up (gate/up)
  const void* packed = nullptr;    // packed part (expert-strided), or nullptr
  void* out = nullptr;             // H (gate/up) or y (down)
  // Contraction split: with ksplit > 1 each tile computes
  // 1/ksplit of the contraction and writes float32 partial sums to `part` instead
  // of `out`: [ksplit][rows][d] for down; for gate/up the gate sums
  // [ksplit][rows][inter] followed by the up sums in the same shape.
  int ksplit = 1;
  float* part = nullptr;
  // int8 codes (launch_ffn_tile_w8): `packed` holds the code tiles, sc0 the row
  // scales of the gate rows [n_exp, inter] (down: of the output columns
  // [n_exp, d]) and sc1 those of the up rows
  const float* sc0 = nullptr;
  const float* sc1 = nullptr;
  // 64-row bf16 tiles: mark the weight loads non-temporal (weights of experts
  // with few rows each, read once per launch, so that they do not push the
  // activation rows every weight tile re-reads out of L2)
  bool nt_weights = false;
  // 256-row gate/up tiles: kSchedInts ints of device memory for round counters
  // (16 ints apart, one per XCD, zero at launch), with which a launch of many
  // rounds runs persistent workgroups that start each round of tiles together;
  // nullptr: one tile per workgroup
  int* rounds = nullptr;
};
// big: 256-row tiles; otherwise 64-row tiles (wide: 96-feature gate/up tiles,
// needing a width divisible by 96, or 256-column down tiles, needing d % 256 == 0)
hipError_t launch_ffn_tile(bool gateup, bool big, int d, const TileSeg& a, const TileSeg* b,
                           hipStream_t st, bool wide = false);
// one projection (gate/up or down) of the routed experts on 64-row tiles (narrow
// or wide) and of one unsplit shared segment on 256-row tiles, in one launch;
// sched: kSchedInts ints of device memory, zero at launch, that the launch uses as
// the XCDs' work counters
constexpr int kSchedInts = 16 * 8;
// down: the shared tiles write float32 partial sums of big.ksplit slices (one or
// more) to big.part, as a sliced segment does; gate/up: big.ksplit == 1
hipError_t launch_ffn_mixed(bool gateup, int d, const TileSeg& small, const TileSeg& big,
                            bool wide, int* sched, hipStream_t st);
// Slices of the shared down projection's contraction in a mixed launch: a shared
// 256-row down tile runs the whole shared intermediate width (5376 for four
// experts of 1344), several times as long as a routed 64-row tile.  Two slices,
// whose float32 partial sums the combine adds, took a 456-token batch's down
// stage from 0.203 to 0.192 ms; three and four slices took 0.202-0.205 ms.
// Slicing the shared gate/up tiles as well (with a SwiGLU pass over the partial
// sums) made that stage slower, 0.353 -> 0.384 ms.
constexpr int kMixedDownSlices = 2;
// shapes the tile kernels cover (96- and 192-feature gate/up tiles, 256-column down tiles)
bool tile_path_ok(int d, int inter);
// 64-row tiles on int8 codes (tiles from `thr` rows up), and the shapes they cover
// (wide: 256-column down tiles; gate/up tiles are always narrow)
hipError_t launch_ffn_tile_w8(bool gateup, int d, const TileSeg& a, const TileSeg* b,
                              hipStream_t st, bool wide = false);
bool tile_path_w8_ok(int d, int inter);
// Contraction slices for a single segment of `rows` rows on tiles of `tile_rows`
// rows with contraction K and `col_tiles` weight tiles per row tile: as many as
// still fit one round of workgroups (planned for 256 CUs), at least 12 stages of
// 64 per slice.  1 = no split, at most kMaxSlices.  Depends on the sizes only.
constexpr int kMaxSlices = 8;
int tile_ksplit(int rows, int K, int col_tiles, int tile_rows = 64);
// output columns of one 64-row down tile, and features of one 64-row gate/up tile,
// narrow or wide
int small_down_cols(bool wide);
int small_gateup_feats(bool wide);
// H = silu(sum of gate partials) * (sum of up partials), slices added in order, bf16
hipError_t launch_swiglu_parts(const float* part, int ksplit, int rows, int inter, void* h,
                               hipStream_t st);

// ---- weight packing (pack.hip) --------------------------------------------
// src1 != nullptr: gate/up pair [n_exp, rows, K] each; else down [n_exp, rows, K]
hipError_t launch_pack(int dtype, const void* src0, const void* src1, int n_exp, int rows, int K,
                       void* dst, hipStream_t st);

// ---- combine (combine.hip) -------------------------------------------------
// shared_part (optional, instead of `shared`): n_part float32 partial sums
// [n_part][T][d] of the shared experts' output, added in slice order
hipError_t launch_combine(int dtype, int T, int K, int d, const void* y_perm,
                          const int32_t* pair_row, const float* gate, const void* shared,
                          const float* shared_part, int n_part, void* y, hipStream_t st);

}  // namespace moge
