// C ABI of the MoGE layer library: host-side validation, workspace carving and
// kernel dispatch on the caller's stream.  No device allocation, no host
// synchronisation, no host reads of device data.
#include <limits.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moge.h"
#include "moge_internal.hpp"
#include "packed_layout.hpp"
#include "w8_layout.hpp"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_stage_events[MOGE_STAGE_EVENTS];
thread_local bool g_record_stages = false;

void mark(int i, hipStream_t st) {
  if (g_record_stages && g_stage_events[i]) (void)hipEventRecord(g_stage_events[i], st);
}

moge_status_t fail(moge_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moge_status_t fail(moge_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moge_status_t ok() {
  g_last_error.clear();
  return MOGE_OK;
}

moge_status_t hip_check(hipError_t e, const char* where) {
  if (e != hipSuccess)
    return fail(MOGE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return MOGE_OK;
}

constexpr int kMaxExperts = 256;
constexpr int kMaxSlots = 64;

int esize(const moge_dims_t* d) { return d->dtype == MOGE_BF16 ? 2 : 4; }

moge_status_t check_dims(const moge_dims_t* d) {
  if (!d) return fail(MOGE_ERR_INVALID_ARG, "dims is NULL");
  if (d->T < 0 || d->d <= 0 || d->N <= 0 || d->M <= 0 || d->k_per_group <= 0 || d->inter <= 0 ||
      d->shared_inter < 0)
    return fail(MOGE_ERR_INVALID_ARG,
                "dims out of range (T=%d d=%d N=%d M=%d k_per_group=%d inter=%d shared_inter=%d)",
                d->T, d->d, d->N, d->M, d->k_per_group, d->inter, d->shared_inter);
  if (d->N % d->M != 0)
    return fail(MOGE_ERR_INVALID_ARG, "N=%d is not a multiple of M=%d", d->N, d->M);
  if (d->k_per_group > d->N / d->M)
    return fail(MOGE_ERR_INVALID_ARG, "k_per_group=%d exceeds the group size N/M=%d",
                d->k_per_group, d->N / d->M);
  if (d->dtype != MOGE_F32 && d->dtype != MOGE_BF16)
    return fail(MOGE_ERR_INVALID_ARG, "dtype=%d is not MOGE_F32 or MOGE_BF16", d->dtype);
  if (d->N > kMaxExperts) return fail(MOGE_ERR_UNSUPPORTED, "N=%d > %d", d->N, kMaxExperts);
  const int K = d->M * d->k_per_group;
  if (K > kMaxSlots) return fail(MOGE_ERR_UNSUPPORTED, "K=M*k_per_group=%d > %d", K, kMaxSlots);
  if (d->d % 32 || d->inter % 32 || d->shared_inter % 32)
    return fail(MOGE_ERR_UNSUPPORTED, "d=%d, inter=%d and shared_inter=%d must be multiples of 32",
                d->d, d->inter, d->shared_inter);
  if ((long long)d->T * K >= (1ll << 31))
    return fail(MOGE_ERR_UNSUPPORTED, "T*K=%lld rows exceed int32", (long long)d->T * K);
  // activation-side buffers are addressed with 32-bit byte offsets
  const long long R = (long long)d->T * K, es = esize(d);
  long long widest = R * d->d;
  if (R * d->inter > widest) widest = R * d->inter;
  if ((long long)d->T * d->shared_inter > widest) widest = (long long)d->T * d->shared_inter;
  // one expert's packed gate/up pair, and the shared experts' (one buffer each)
  if (2ll * d->inter * d->d > widest) widest = 2ll * d->inter * d->d;
  if (2ll * d->shared_inter * d->d > widest) widest = 2ll * d->shared_inter * d->d;
  if (widest * es > 0xFFFFFFFFll)
    return fail(MOGE_ERR_UNSUPPORTED, "an activation or expert buffer exceeds 4 GiB (%lld bytes)",
                widest * es);
  return MOGE_OK;
}

moge_status_t check_ptr(const void* p, size_t align, const char* name, bool required) {
  if (!p) {
    if (required) return fail(MOGE_ERR_INVALID_ARG, "%s is NULL", name);
    return MOGE_OK;
  }
  if (reinterpret_cast<uintptr_t>(p) % align)
    return fail(MOGE_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return MOGE_OK;
}

#define CHECK(expr)                         \
  do {                                      \
    const moge_status_t s_ = (expr);        \
    if (s_ != MOGE_OK) return s_;           \
  } while (0)

// The int8 experts: bf16 activations, and contraction widths made of whole
// 64-element code tiles.
moge_status_t check_w8_dims(const moge_dims_t* d) {
  CHECK(check_dims(d));
  if (d->dtype != MOGE_BF16)
    return fail(MOGE_ERR_UNSUPPORTED, "int8 expert weights take bf16 activations (dtype=%d)",
                d->dtype);
  if (d->d % 64 || d->inter % 64 || d->shared_inter % 64)
    return fail(MOGE_ERR_UNSUPPORTED,
                "int8 experts need d=%d, inter=%d and shared_inter=%d to be multiples of 64", d->d,
                d->inter, d->shared_inter);
  return MOGE_OK;
}

// ---------------------------------------------------------------------------
// workspace layout (256-byte aligned regions)
// ---------------------------------------------------------------------------
struct Plan {
  size_t partial, idx, gate, blk_cnt, blk_base, counts, offsets, gcounts, sorted_pair, pair_row,
      h, hs, y_perm, sh, sh_part, sched, total;
  int ksplit;
};

// Contraction slices of the shared experts' tile launches (gate/up, down); 1 = not
// split.  A single segment of a few dozen rows makes too few tiles to cover the
// CUs, so its contraction is split and the float32 partial sums are added
// afterwards (gate/up: by k_swiglu_parts, down: by the combine).  dn_parts: the
// down projection writes float32 partial sums even as one slice (the mixed
// launches' shared tiles always do).
struct SharedSplit {
  int gu = 1, dn = 1;
  bool dn_parts = false;
  bool down_parts() const { return dn > 1 || dn_parts; }
};

bool tiles_ok_for(const moge_dims_t* d) {
  return d->dtype == MOGE_BF16 && moge::tile_path_ok(d->d, d->inter) &&
         (d->shared_inter == 0 || moge::tile_path_ok(d->d, d->shared_inter));
}

bool w8_tiles_ok_for(const moge_dims_t* d) {
  return moge::tile_path_w8_ok(d->d, d->inter) &&
         (d->shared_inter == 0 || moge::tile_path_w8_ok(d->d, d->shared_inter));
}

// The 64-row tiles are wide (96 gate/up features, 256 down columns) when the routed
// experts can fill several rounds of them: a mean of at least kStreamMaxRows rows
// per expert (R / N).  Below that the launch holds mostly the split shared
// segment, one round, which narrow tiles spread over more CUs.  The widths must
// divide into wide tiles (the routed and shared widths by 96 features, d by 256).
bool many_small_tiles(long long R, int N) {
  return N > 0 && (double)R / N >= moge::kStreamMaxRows;
}
bool wide_down(long long R, int N, int d) {
  return many_small_tiles(R, N) && d % moge::small_down_cols(true) == 0;
}
bool wide_gateup(long long R, int N, int inter, int shared_inter) {
  const int f = moge::small_gateup_feats(true);
  return many_small_tiles(R, N) && inter % f == 0 && shared_inter % f == 0;
}

// Row ranges of the routed experts: the streaming kernels take experts with at
// most `stream_max` rows, the 64-row tiles those up to `small_max`, the 256-row
// tiles the rest.  Each expert's kernel is chosen on the device from its row
// count, and the host cannot see the counts, so every range gets a launch, and a
// launch that finds no expert still costs about 4 us.  The mean rows per expert
// (R / N) is known on the host; a range that is unlikely to hold an expert at that
// mean joins its neighbour (any kernel handles any row count):
//   mean >= 1.5 * kStreamMaxRows:    experts of up to kStreamMaxRows rows take the
//                                    64-row tiles (no streaming launch);
//   mean <= kSmallTileMaxRows / 2:   experts above kSmallTileMaxRows rows stay on
//                                    64-row tiles (no 256-row launch);
//   mean >= 2 * kSmallTileMaxRows:   every routed expert takes 256-row tiles.
struct RoutedRanges {
  int stream_max, small_max;
};
RoutedRanges routed_ranges(long long R, int N, bool big_tiles) {
  RoutedRanges r{moge::kStreamMaxRows, big_tiles ? moge::kSmallTileMaxRows : INT_MAX};
  const double mean = N > 0 ? (double)R / N : 0.0;
  if (mean >= 1.5 * moge::kStreamMaxRows) r.stream_max = 0;
  if (big_tiles && mean <= moge::kSmallTileMaxRows / 2) r.small_max = INT_MAX;
  if (big_tiles && mean >= 2.0 * moge::kSmallTileMaxRows) r.stream_max = r.small_max = 0;
  return r;
}

// The launches that mix tile shapes (routed experts on 64-row tiles beside the
// shared segment on 256-row tiles, moge::launch_ffn_mixed) serve batches whose
// routed experts all take 64-row tiles and whose shared segment is above the
// 64-row tiles' limit in both projections: a mean of 48 to 64 rows per expert.
bool mixed_regime(bool tiles_ok, const RoutedRanges& rr, int shared_rows) {
  return tiles_ok && rr.stream_max == 0 && rr.small_max == INT_MAX &&
         shared_rows > moge::kSharedSmallGateUpRows && shared_rows > moge::kSharedSmallDownRows;
}

// w8: the int8 layer, whose shared segment takes 64-row tiles at every size above
// the streaming limit
SharedSplit shared_split(const moge_dims_t* d, bool w8) {
  SharedSplit s;
  const int T = d->T, Is = d->shared_inter;
  if (Is == 0 || T <= moge::kSharedStreamMaxRows) return s;
  if (w8 ? !w8_tiles_ok_for(d) : !tiles_ok_for(d)) return s;
  // 64-row tiles: small_gateup_feats features (gate/up) or small_down_cols columns
  // (down) per tile, narrow or wide as the launch will be; 256-row tiles: 96
  // features or 256 columns
  const long long R = (long long)T * d->M * d->k_per_group;
  // the bf16 layer's mixed launches run the shared gate/up unsplit and the shared
  // down on kMixedDownSlices slices (one where they do not divide its stages),
  // as float32 partial sums either way
  if (!w8 && mixed_regime(true, routed_ranges(R, d->N, true), T)) {
    if ((Is / 64) % moge::kMixedDownSlices == 0) s.dn = moge::kMixedDownSlices;
    s.dn_parts = true;
    return s;
  }
  if (w8 || T <= moge::kSharedSmallGateUpRows)
    s.gu = moge::tile_ksplit(
        T, d->d, Is / moge::small_gateup_feats(!w8 && wide_gateup(R, d->N, d->inter, Is)), 64);
  else
    s.gu = moge::tile_ksplit(T, d->d, Is / 96, 256);
  if (w8 || T <= moge::kSharedSmallDownRows)
    s.dn = moge::tile_ksplit(T, Is, d->d / moge::small_down_cols(wide_down(R, d->N, d->d)), 64);
  else
    s.dn = moge::tile_ksplit(T, Is, d->d / 256, 256);
  return s;
}

// float32 partial-sum bytes a split needs (gate/up and down use it in turn)
size_t split_part_bytes(const moge_dims_t* d, const SharedSplit& ss) {
  size_t part = 0;
  if (ss.gu > 1) part = (size_t)2 * ss.gu * d->T * d->shared_inter * 4;
  if (ss.down_parts() && (size_t)ss.dn * d->T * d->d * 4 > part)
    part = (size_t)ss.dn * d->T * d->d * 4;
  return part;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Plan make_plan(const moge_dims_t* d) {
  Plan p{};
  const size_t T = d->T, N = d->N, M = d->M, K = (size_t)d->M * d->k_per_group, R = T * K;
  const size_t es = esize(d), nblk = moge::perm_blocks(d->T);
  p.ksplit = moge::router_ksplit(d->dtype, d->T, d->d, d->N);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes > 0 ? bytes : 1);
    return at;
  };
  p.partial = take((size_t)p.ksplit * T * N * 4);
  p.idx = take(T * K * 4);
  p.gate = take(T * K * 4);
  p.blk_cnt = take(nblk * N * 4);
  p.blk_base = take(nblk * N * 4);
  p.counts = take(N * 4);
  p.offsets = take((N + 1) * 4);
  p.gcounts = take(M * 4);
  p.sorted_pair = take(R * 4);
  p.pair_row = take(R * 4);
  p.h = take(R * (size_t)d->inter * es);
  p.hs = take(T * (size_t)d->shared_inter * es);
  p.y_perm = take(R * (size_t)d->d * es);
  p.sh = take(T * (size_t)d->d * es);
  // the bf16 and the int8 layer share the workspace layout
  const size_t part_bf16 = split_part_bytes(d, shared_split(d, false));
  const size_t part_w8 = d->dtype == MOGE_BF16 ? split_part_bytes(d, shared_split(d, true)) : 0;
  p.sh_part = take(part_bf16 > part_w8 ? part_bf16 : part_w8);
  p.sched = take(2 * moge::kSchedInts * 4);   // gate/up's counters, then down's
  p.total = o;
  return p;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

moge_status_t check_ws(const moge_dims_t* d, void* ws, size_t ws_bytes, Plan* plan) {
  *plan = make_plan(d);
  if (!ws) return fail(MOGE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan->total);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(MOGE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (ws_bytes < plan->total)
    return fail(MOGE_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, plan->total);
  return MOGE_OK;
}

// The tile-path view of a streaming segment: gate/up reads x (or x_perm) and
// writes H; down reads H and writes y.
moge::TileSeg tile_view(const moge::FfnSeg& f, bool gateup) {
  moge::TileSeg t;
  t.n_exp = f.n_exp;
  t.inter = f.inter;
  t.thr = f.thr;
  t.offsets = f.offsets;
  t.rows = f.rows;
  // experts with their own row ranges (the routed experts): each one's weights
  // are read once per launch.  The shared segment (one expert, every token) keeps
  // cached loads: a 64-token decode batch measured slower with the hint there.
  t.nt_weights = f.offsets != nullptr;
  if (gateup) {
    t.x = f.x;
    t.x_rows = f.x_rows;
    t.row_src = f.row_src;
    t.row_div = f.row_div;
    t.w0 = f.w_gate;
    t.w1 = f.w_up;
    t.packed = f.p_gu;
    t.out = f.h;
  } else {
    t.x = f.h;
    t.x_rows = f.rows;
    t.w0 = f.w_down;
    t.packed = f.p_down;
    t.out = f.y;
  }
  return t;
}

// Both projections of up to two segments.  The routed experts go to the streaming,
// 64-row and 256-row kernels by the ranges routed_ranges gives; the shared segment
// has its own limits (kSharedStreamMaxRows, kSharedSmallGateUpRows,
// kSharedSmallDownRows).  A tile launch is made only when some expert can fall in
// its range (an expert never has more rows than the batch has tokens).
// split: contraction slices for the shared segment's tiles, with sh_part the
// float32 partial-sum region (used when a slice count is above 1, and by the
// mixed launches' shared down tiles whatever their count).
// sched: 2 x kSchedInts ints, zero at the call, for the work counters of the
// gate/up launch and then of the down launch; nullptr: launches that need none.
moge_status_t run_ffn(int dtype, int d, int T, moge::FfnSeg& routed, moge::FfnSeg* sh,
                      hipStream_t st, bool marks, SharedSplit split = SharedSplit{},
                      float* sh_part = nullptr, int* sched = nullptr) {
  // the tile path covers bf16 and its tile shapes; everything else streams
  const bool tiles_ok = dtype == MOGE_BF16 && moge::tile_path_ok(d, routed.inter) &&
                        (!sh || moge::tile_path_ok(d, sh->inter));
  const RoutedRanges rr = routed_ranges(routed.rows, routed.n_exp, true);
  const int thr = tiles_ok ? rr.stream_max : INT_MAX;
  const int sh_thr = tiles_ok ? moge::kSharedStreamMaxRows : INT_MAX;
  const int thr_big = rr.small_max;
  const bool wide_gu = wide_gateup(routed.rows, routed.n_exp, routed.inter, sh ? sh->inter : 0);
  const bool wide_dn = wide_down(routed.rows, routed.n_exp, d);
  routed.thr = thr;
  if (sh) sh->thr = sh_thr;
  const bool sh_stream = sh && sh->rows <= sh_thr;
  // the streaming launches, with the routed experts only when their range is open
  moge::FfnSeg rs = routed;
  if (thr == 0) rs.n_exp = 0;
  const bool stream_launch = rs.n_exp > 0 || sh_stream;
  // tile launches: routed experts with lo < rows <= hi, the shared segment with
  // sh_lo < rows <= sh_hi
  struct Range { int lo, hi, sh_lo, sh_hi; bool big; };
  // a batch whose routed experts all take 64-row tiles (none streams, none takes
  // 256-row tiles) while the shared segment takes 256-row tiles in both
  // projections: one launch per projection for both, with the shared gate/up
  // contraction unsplit (the routed tiles fill the CUs beside it) and the shared
  // down one as float32 partial sums of kMixedDownSlices slices (or one)
  const bool mixed = sched && mixed_regime(tiles_ok, rr, sh ? sh->rows : 0);
  for (int gateup = 1; gateup >= 0; --gateup) {
    const int sh_big = gateup ? moge::kSharedSmallGateUpRows : moge::kSharedSmallDownRows;
    const Range ranges[2] = {{thr, thr_big, sh_thr, sh_big, false},
                             {thr_big, INT_MAX, sh_big, INT_MAX, true}};
    if (stream_launch && gateup)
      CHECK(hip_check(moge::launch_ffn_gateup(dtype, d, rs, sh_stream ? sh : nullptr, st),
                      "expert gate/up"));
    else if (stream_launch)
      CHECK(hip_check(moge::launch_ffn_down(dtype, d, rs, sh_stream ? sh : nullptr, st),
                      "expert down"));
    if (mixed) {
      moge::TileSeg a = tile_view(routed, gateup);
      a.thr = 0;
      a.thr_hi = INT_MAX;
      moge::TileSeg b = tile_view(*sh, gateup);
      b.thr = 0;
      b.thr_hi = INT_MAX;
      if (!gateup && split.down_parts() && sh_part) {
        b.ksplit = split.dn;
        b.part = sh_part;
      }
      CHECK(hip_check(moge::launch_ffn_mixed(gateup, d, a, b, gateup ? wide_gu : wide_dn,
                                             sched + (gateup ? 0 : moge::kSchedInts), st),
                      gateup ? "expert gate/up tiles (routed and shared)"
                             : "expert down tiles (routed and shared)"));
      if (marks) mark(gateup ? 4 : 5, st);
      continue;
    }
    for (const Range& rg : ranges) {
      const bool routed_here = tiles_ok && T > rg.lo && rg.lo < rg.hi;
      const bool sh_here = tiles_ok && sh && sh->rows > rg.sh_lo && sh->rows <= rg.sh_hi;
      if (!routed_here && !sh_here) continue;
      moge::TileSeg a = tile_view(routed, gateup);
      a.thr = rg.lo;
      a.thr_hi = rg.hi;
      if (!routed_here) a.n_exp = 0;
      moge::TileSeg b;
      const int ks = gateup ? split.gu : split.dn;
      const bool sliced = sh_here && ks > 1 && sh_part;
      if (sh_here) {
        b = tile_view(*sh, gateup);
        b.thr = rg.sh_lo;
        b.thr_hi = rg.sh_hi;
        if (sliced) {
          b.ksplit = ks;
          b.part = sh_part;
        }
      }
      const char* what = gateup ? "expert gate/up tiles" : "expert down tiles";
      if (sliced && rg.big) {
        // sliced 256-row tiles are an instantiation of their own: the routed
        // experts of this range go in a plain launch first
        if (routed_here) CHECK(hip_check(moge::launch_ffn_tile(gateup, true, d, a, nullptr, st), what));
        CHECK(hip_check(moge::launch_ffn_tile(gateup, true, d, b, nullptr, st), what));
      } else {
        // a gate/up launch of many rounds of 256-row tiles keeps its rounds with
        // these counters
        if (rg.big && gateup) a.rounds = sched;
        CHECK(hip_check(moge::launch_ffn_tile(gateup, rg.big, d, a, sh_here ? &b : nullptr, st,
                                              gateup ? wide_gu : wide_dn),
                        what));
      }
      if (sliced && gateup)
        CHECK(hip_check(moge::launch_swiglu_parts(sh_part, ks, sh->rows, sh->inter, sh->h, st),
                        "shared SwiGLU of the slices"));
    }
    if (marks) mark(gateup ? 4 : 5, st);
  }
  return MOGE_OK;
}

// The tile-path view of an int8 segment: code tiles and row scales.
moge::TileSeg tile_view_w8(const moge::FfnSeg& f, bool gateup) {
  moge::TileSeg t = tile_view(f, gateup);
  t.packed = gateup ? f.p_gu : f.p_down;
  t.sc0 = gateup ? f.sc_gate : f.sc_down;
  t.sc1 = gateup ? f.sc_up : nullptr;
  return t;
}

// Weight-only int8 experts: experts with at most kStreamMaxRows rows (the shared
// segment: kSharedStreamMaxRows) stream their codes, unless the mean rows per
// expert folds that range into the tiles; larger ones take the int8 64-row tiles
// (wide down tiles when the routed experts fill several rounds), the shared
// segment with its contraction split when it is small.  Without a tile shape for
// the sizes every expert streams.
moge_status_t run_ffn_w8(int d, int T, moge::FfnSeg& routed, moge::FfnSeg* sh, hipStream_t st,
                         bool marks, SharedSplit split, float* sh_part) {
  const bool tiles = moge::tile_path_w8_ok(d, routed.inter) &&
                     (!sh || moge::tile_path_w8_ok(d, sh->inter));
  routed.thr = tiles ? routed_ranges(routed.rows, routed.n_exp, false).stream_max : INT_MAX;
  if (sh) sh->thr = tiles ? moge::kSharedStreamMaxRows : INT_MAX;
  const bool sh_stream = sh && sh->rows <= sh->thr;
  moge::FfnSeg rs = routed;
  if (routed.thr == 0) rs.n_exp = 0;
  const bool stream_launch = rs.n_exp > 0 || sh_stream;
  for (int gateup = 1; gateup >= 0; --gateup) {
    if (stream_launch && gateup)
      CHECK(hip_check(moge::launch_ffn_gateup_w8(d, rs, sh_stream ? sh : nullptr, st),
                      "int8 expert gate/up"));
    else if (stream_launch)
      CHECK(hip_check(moge::launch_ffn_down_w8(d, rs, sh_stream ? sh : nullptr, st),
                      "int8 expert down"));
    const bool routed_here = tiles && T > routed.thr;
    const bool sh_here = tiles && sh && !sh_stream;
    if (routed_here || sh_here) {
      moge::TileSeg a = tile_view_w8(routed, gateup);
      a.thr = routed.thr;
      if (!routed_here) a.n_exp = 0;
      moge::TileSeg b;
      const int ks = gateup ? split.gu : split.dn;
      const bool sliced = sh_here && ks > 1 && sh_part;
      if (sh_here) {
        b = tile_view_w8(*sh, gateup);
        b.thr = sh->thr;
        if (sliced) {
          b.ksplit = ks;
          b.part = sh_part;
        }
      }
      CHECK(hip_check(moge::launch_ffn_tile_w8(gateup, d, a, sh_here ? &b : nullptr, st,
                                               !gateup && wide_down(routed.rows, routed.n_exp, d)),
                      gateup ? "int8 expert gate/up tiles" : "int8 expert down tiles"));
      if (sliced && gateup)
        CHECK(hip_check(moge::launch_swiglu_parts(sh_part, ks, sh->rows, sh->inter, sh->h, st),
                        "shared SwiGLU of the slices"));
    }
    if (marks) mark(gateup ? 4 : 5, st);
  }
  return MOGE_OK;
}

struct Weights {
  const void *gate = nullptr, *up = nullptr, *down = nullptr;        // row-major routed
  const void *s_gate = nullptr, *s_up = nullptr, *s_down = nullptr;  // row-major shared
  const void *p_gu = nullptr, *p_down = nullptr;                     // packed routed
  const void *ps_gu = nullptr, *ps_down = nullptr;                   // packed shared
  bool w8 = false;  // p_* / ps_* hold int8 code tiles with the scales below
  const float *sc_gate = nullptr, *sc_up = nullptr, *sc_down = nullptr;     // routed
  const float *ssc_gate = nullptr, *ssc_up = nullptr, *ssc_down = nullptr;  // shared
};

// The whole layer on one stream; `w` holds either row-major or packed weights
// (pointers already checked by the caller).
moge_status_t layer_impl(const moge_dims_t* dims, const void* x, const void* w_router,
                         const float* router_bias, const Weights& w, const float* logits_in,
                         void* y, float* logits_out, int32_t* topk_idx_out, float* topk_gate_out,
                         int32_t* group_counts_out, void* ws, size_t ws_bytes, void* stream) {
  const bool shared = dims->shared_inter > 0;
  CHECK(check_ptr(x, 16, "x", true));
  CHECK(check_ptr(logits_in, 4, "logits_in", false));
  CHECK(check_ptr(w_router, 16, "w_router", logits_in == nullptr));
  CHECK(check_ptr(router_bias, 4, "router_bias", false));
  CHECK(check_ptr(y, 16, "y", true));
  CHECK(check_ptr(logits_out, 4, "logits_out", false));
  CHECK(check_ptr(topk_idx_out, 4, "topk_idx_out", false));
  CHECK(check_ptr(topk_gate_out, 4, "topk_gate_out", false));
  CHECK(check_ptr(group_counts_out, 4, "group_counts_out", false));
  Plan p;
  CHECK(check_ws(dims, ws, ws_bytes, &p));
  if (dims->T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = dims->T, N = dims->N, M = dims->M, kp = dims->k_per_group, K = M * kp;
  const int R = T * K;

  mark(0, st);
  // S0 router scores (split contraction, partial sums added by the routing kernel)
  const float* scores = logits_in;
  const float* bias = nullptr;
  int ksplit = 1;
  if (!logits_in) {
    float* partial = at<float>(ws, p.partial);
    CHECK(hip_check(moge::launch_router_scores(dims->dtype, x, w_router, T, dims->d, N, p.ksplit,
                                               partial, st),
                    "router scores"));
    scores = partial;
    bias = router_bias;
    ksplit = p.ksplit;
  }
  mark(1, st);
  // S1+S2 softmax and grouped top-K'
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, p.idx);
  float* gate = topk_gate_out ? topk_gate_out : at<float>(ws, p.gate);
  // (the routing kernel also zeroes the expert launches' work counters)
  CHECK(hip_check(moge::launch_route(scores, ksplit, T, N, M, kp, bias, logits_out, nullptr, idx,
                                     gate, st, at<int>(ws, p.sched), 2 * moge::kSchedInts),
                  "route"));
  mark(2, st);
  // S3 permutation (the FFN gathers its rows from x through sorted_pair)
  int32_t* gcounts = group_counts_out ? group_counts_out : at<int32_t>(ws, p.gcounts);
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* sorted_pair = at<int32_t>(ws, p.sorted_pair);
  int32_t* pair_row = at<int32_t>(ws, p.pair_row);
  CHECK(hip_check(moge::launch_permute(idx, T, K, N, M, at<int32_t>(ws, p.blk_cnt),
                                       at<int32_t>(ws, p.blk_base), at<int32_t>(ws, p.counts),
                                       offsets, gcounts, sorted_pair, pair_row, st),
                  "permute"));
  mark(3, st);
  // S4-S6 routed and shared SwiGLU experts, one launch per projection
  moge::FfnSeg routed;
  routed.x = x;
  routed.x_rows = T;
  routed.row_src = sorted_pair;
  routed.row_div = K;
  routed.offsets = offsets;
  routed.rows = R;
  routed.n_exp = N;
  routed.inter = dims->inter;
  routed.w_gate = w.gate;
  routed.w_up = w.up;
  routed.w_down = w.down;
  routed.p_gu = w.p_gu;
  routed.p_down = w.p_down;
  routed.sc_gate = w.sc_gate;
  routed.sc_up = w.sc_up;
  routed.sc_down = w.sc_down;
  routed.h = at<char>(ws, p.h);
  routed.y = at<char>(ws, p.y_perm);
  moge::FfnSeg sh;
  if (shared) {
    sh.x = x;
    sh.x_rows = T;
    sh.rows = T;
    sh.n_exp = 1;
    sh.inter = dims->shared_inter;
    sh.w_gate = w.s_gate;
    sh.w_up = w.s_up;
    sh.w_down = w.s_down;
    sh.p_gu = w.ps_gu;
    sh.p_down = w.ps_down;
    sh.sc_gate = w.ssc_gate;
    sh.sc_up = w.ssc_up;
    sh.sc_down = w.ssc_down;
    sh.h = at<char>(ws, p.hs);
    sh.y = at<char>(ws, p.sh);
  }
  const SharedSplit split = shared_split(dims, w.w8);
  float* const sh_part = at<float>(ws, p.sh_part);
  if (w.w8)
    CHECK(run_ffn_w8(dims->d, T, routed, shared ? &sh : nullptr, st, true, split, sh_part));
  else
    CHECK(run_ffn(dims->dtype, dims->d, T, routed, shared ? &sh : nullptr, st, true, split,
                  sh_part, at<int>(ws, p.sched)));
  // S7 combine (the shared term as the slices' partial sums when its down
  // projection was split)
  const bool dn_parts = shared && split.down_parts();
  CHECK(hip_check(moge::launch_combine(dims->dtype, T, K, dims->d, routed.y, pair_row, gate,
                                       shared && !dn_parts ? sh.y : nullptr,
                                       dn_parts ? sh_part : nullptr, dn_parts ? split.dn : 0, y,
                                       st),
                  "combine"));
  mark(6, st);
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// The workspace of moge_layer_forward_packed_noalloc: a fixed device array, for
// callers that cannot allocate device memory or pass a workspace.  Every GPU that
// runs the library holds its own copy until the process ends.  In host code the
// array's name is only a stand-in for the symbol, not a device address: its
// address on a device comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOGE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the first
// call on each device).
moge_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  CHECK(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOGE_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    CHECK(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                    "hipGetSymbolAddress(scratch)"));
    if (!p || reinterpret_cast<uintptr_t>(p) % 256)
      return fail(MOGE_ERR_HIP, "scratch array of device %d at %p is not 256-byte aligned", dev,
                  p);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOGE_OK;
}

}  // namespace

extern "C" {

int32_t moge_abi_version(void) { return 1; }

moge_status_t moge_set_stage_events(void* const* events, int32_t n_events) {
  if (!events || n_events == 0) {
    g_record_stages = false;
    return ok();
  }
  if (n_events != MOGE_STAGE_EVENTS)
    return fail(MOGE_ERR_INVALID_ARG, "n_events=%d, expected %d", n_events, MOGE_STAGE_EVENTS);
  for (int i = 0; i < MOGE_STAGE_EVENTS; ++i) g_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  g_record_stages = true;
  return ok();
}

const char* moge_last_error(void) { return g_last_error.c_str(); }

size_t moge_workspace_size(const moge_dims_t* dims) {
  const std::string saved = g_last_error;
  const moge_status_t s = check_dims(dims);
  g_last_error = saved;
  if (s != MOGE_OK) return 0;
  return make_plan(dims).total;
}

moge_status_t moge_route(const moge_dims_t* dims, const float* logits, float* probs,
                         int32_t* topk_idx, float* topk_gate, void* stream) {
  CHECK(check_dims(dims));
  CHECK(check_ptr(logits, 4, "logits", true));
  CHECK(check_ptr(probs, 4, "probs", false));
  CHECK(check_ptr(topk_idx, 4, "topk_idx", true));
  CHECK(check_ptr(topk_gate, 4, "topk_gate", true));
  if (dims->T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(hip_check(moge::launch_route(logits, 1, dims->T, dims->N, dims->M, dims->k_per_group,
                                     nullptr, nullptr, probs, topk_idx, topk_gate, st),
                  "moge_route"));
  return ok();
}

moge_status_t moge_permute(const moge_dims_t* dims, const int32_t* topk_idx, const void* x,
                           int32_t* counts, int32_t* offsets, int32_t* group_counts,
                           int32_t* sorted_pair, int32_t* pair_row, void* x_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  CHECK(check_dims(dims));
  CHECK(check_ptr(topk_idx, 4, "topk_idx", true));
  CHECK(check_ptr(counts, 4, "counts", true));
  CHECK(check_ptr(offsets, 4, "offsets", true));
  CHECK(check_ptr(group_counts, 4, "group_counts", true));
  CHECK(check_ptr(sorted_pair, 4, "sorted_pair", true));
  CHECK(check_ptr(pair_row, 4, "pair_row", true));
  CHECK(check_ptr(x_perm, 16, "x_perm", false));
  CHECK(check_ptr(x, 16, "x", x_perm != nullptr));
  Plan p;
  CHECK(check_ws(dims, ws, ws_bytes, &p));
  if (dims->T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int K = dims->M * dims->k_per_group;
  CHECK(hip_check(moge::launch_permute(topk_idx, dims->T, K, dims->N, dims->M,
                                       at<int32_t>(ws, p.blk_cnt), at<int32_t>(ws, p.blk_base),
                                       counts, offsets, group_counts, sorted_pair, pair_row, st),
                  "moge_permute"));
  if (x_perm)
    CHECK(hip_check(moge::launch_gather_rows(dims->dtype, x, sorted_pair, offsets + dims->N,
                                             dims->T * K, K, dims->d, x_perm, st),
                    "moge_permute gather"));
  return ok();
}

moge_status_t moge_expert_ffn(const moge_dims_t* dims, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                              void* stream) {
  CHECK(check_dims(dims));
  CHECK(check_ptr(x_perm, 16, "x_perm", true));
  CHECK(check_ptr(offsets, 4, "offsets", true));
  CHECK(check_ptr(w_gate, 16, "w_gate", true));
  CHECK(check_ptr(w_up, 16, "w_up", true));
  CHECK(check_ptr(w_down, 16, "w_down", true));
  CHECK(check_ptr(y_perm, 16, "y_perm", true));
  Plan p;
  CHECK(check_ws(dims, ws, ws_bytes, &p));
  if (dims->T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int K = dims->M * dims->k_per_group;
  moge::FfnSeg g;
  g.x = x_perm;
  g.x_rows = dims->T * K;
  g.offsets = offsets;
  g.rows = dims->T * K;
  g.n_exp = dims->N;
  g.inter = dims->inter;
  g.w_gate = w_gate;
  g.w_up = w_up;
  g.w_down = w_down;
  g.h = at<char>(ws, p.h);
  g.y = y_perm;
  CHECK(run_ffn(dims->dtype, dims->d, dims->T, g, nullptr, st, false));
  return ok();
}

moge_status_t moge_combine(const moge_dims_t* dims, const void* y_perm, const int32_t* pair_row,
                           const float* topk_gate, const void* shared_out, void* y,
                           void* stream) {
  CHECK(check_dims(dims));
  CHECK(check_ptr(y_perm, 16, "y_perm", true));
  CHECK(check_ptr(pair_row, 4, "pair_row", true));
  CHECK(check_ptr(topk_gate, 4, "topk_gate", true));
  CHECK(check_ptr(shared_out, 16, "shared_out", false));
  CHECK(check_ptr(y, 16, "y", true));
  if (dims->T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  CHECK(hip_check(moge::launch_combine(dims->dtype, dims->T, dims->M * dims->k_per_group, dims->d,
                                       y_perm, pair_row, topk_gate, shared_out, nullptr, 0, y, st),
                  "moge_combine"));
  return ok();
}

moge_status_t moge_layer_forward(const moge_dims_t* dims, const void* x, const void* w_router,
                                 const float* router_bias, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* ws_gate, const void* ws_up,
                                 const void* ws_down, const float* logits_in, void* y,
                                 float* logits_out, int32_t* topk_idx_out, float* topk_gate_out,
                                 int32_t* group_counts_out, void* ws, size_t ws_bytes,
                                 void* stream) {
  CHECK(check_dims(dims));
  const bool shared = dims->shared_inter > 0;
  CHECK(check_ptr(w_gate, 16, "w_gate", true));
  CHECK(check_ptr(w_up, 16, "w_up", true));
  CHECK(check_ptr(w_down, 16, "w_down", true));
  CHECK(check_ptr(ws_gate, 16, "ws_gate", shared));
  CHECK(check_ptr(ws_up, 16, "ws_up", shared));
  CHECK(check_ptr(ws_down, 16, "ws_down", shared));
  Weights w;
  w.gate = w_gate;
  w.up = w_up;
  w.down = w_down;
  w.s_gate = ws_gate;
  w.s_up = ws_up;
  w.s_down = ws_down;
  return layer_impl(dims, x, w_router, router_bias, w, logits_in, y, logits_out, topk_idx_out,
                    topk_gate_out, group_counts_out, ws, ws_bytes, stream);
}

size_t moge_packed_weights_size(const moge_dims_t* dims) {
  const std::string saved = g_last_error;
  const moge_status_t s = check_dims(dims);
  g_last_error = saved;
  if (s != MOGE_OK) return 0;
  return moge::packed_parts(dims->d, dims->N, dims->inter, dims->shared_inter, esize(dims)).total;
}

moge_status_t moge_pack_weights(const moge_dims_t* dims, const void* w_gate, const void* w_up,
                                const void* w_down, const void* ws_gate, const void* ws_up,
                                const void* ws_down, void* packed, size_t packed_bytes,
                                void* stream) {
  CHECK(check_dims(dims));
  const bool shared = dims->shared_inter > 0;
  CHECK(check_ptr(w_gate, 16, "w_gate", true));
  CHECK(check_ptr(w_up, 16, "w_up", true));
  CHECK(check_ptr(w_down, 16, "w_down", true));
  CHECK(check_ptr(ws_gate, 16, "ws_gate", shared));
  CHECK(check_ptr(ws_up, 16, "ws_up", shared));
  CHECK(check_ptr(ws_down, 16, "ws_down", shared));
  CHECK(check_ptr(packed, 256, "packed", true));
  const moge::PackedParts pp =
      moge::packed_parts(dims->d, dims->N, dims->inter, dims->shared_inter, esize(dims));
  if (packed_bytes < pp.total)
    return fail(MOGE_ERR_INVALID_ARG, "packed buffer has %zu bytes, need %zu", packed_bytes,
                pp.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* dst = static_cast<char*>(packed);
  const int dt = dims->dtype, d = dims->d, N = dims->N, I = dims->inter, Is = dims->shared_inter;
  CHECK(hip_check(moge::launch_pack(dt, w_gate, w_up, N, I, d, dst + pp.routed_gu, st),
                  "pack routed gate/up"));
  CHECK(hip_check(moge::launch_pack(dt, w_down, nullptr, N, d, I, dst + pp.routed_down, st),
                  "pack routed down"));
  if (shared) {
    CHECK(hip_check(moge::launch_pack(dt, ws_gate, ws_up, 1, Is, d, dst + pp.shared_gu, st),
                    "pack shared gate/up"));
    CHECK(hip_check(moge::launch_pack(dt, ws_down, nullptr, 1, d, Is, dst + pp.shared_down, st),
                    "pack shared down"));
  }
  return ok();
}

moge_status_t moge_layer_forward_packed(const moge_dims_t* dims, const void* x,
                                        const void* w_router, const float* router_bias,
                                        const void* packed, const float* logits_in, void* y,
                                        float* logits_out, int32_t* topk_idx_out,
                                        float* topk_gate_out, int32_t* group_counts_out,
                                        void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_dims(dims));
  CHECK(check_ptr(packed, 256, "packed", true));
  const moge::PackedParts pp =
      moge::packed_parts(dims->d, dims->N, dims->inter, dims->shared_inter, esize(dims));
  const char* base = static_cast<const char*>(packed);
  Weights w;
  w.p_gu = base + pp.routed_gu;
  w.p_down = base + pp.routed_down;
  if (dims->shared_inter > 0) {
    w.ps_gu = base + pp.shared_gu;
    w.ps_down = base + pp.shared_down;
  }
  return layer_impl(dims, x, w_router, router_bias, w, logits_in, y, logits_out, topk_idx_out,
                    topk_gate_out, group_counts_out, ws, ws_bytes, stream);
}

moge_status_t moge_layer_forward_packed_noalloc(const moge_dims_t* dims, const void* x,
                                                const void* w_router, const float* router_bias,
                                                const void* packed, const float* logits_in,
                                                void* y, float* logits_out,
                                                int32_t* topk_idx_out, float* topk_gate_out,
                                                int32_t* group_counts_out, void* stream) {
  CHECK(check_dims(dims));
  const size_t need = make_plan(dims).total;
  if (need > MOGE_NOALLOC_SCRATCH_BYTES)
    return fail(MOGE_ERR_UNSUPPORTED,
                "these dims need %zu bytes of workspace; the fixed scratch array holds %zu "
                "(T=%d is too large for moge_layer_forward_packed_noalloc: pass a workspace to "
                "moge_layer_forward_packed)",
                need, (size_t)MOGE_NOALLOC_SCRATCH_BYTES, dims->T);
  // the scratch address is per device: the stream must belong to the current one
  int cur = -1, sdev = -1;
  CHECK(hip_check(hipGetDevice(&cur), "hipGetDevice"));
  CHECK(hip_check(hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev),
                  "hipStreamGetDevice"));
  if (sdev != cur)
    return fail(MOGE_ERR_INVALID_ARG,
                "the stream belongs to device %d but device %d is current", sdev, cur);
  void* ws = nullptr;
  CHECK(scratch_on_current_device(&ws));
  return moge_layer_forward_packed(dims, x, w_router, router_bias, packed, logits_in, y,
                                   logits_out, topk_idx_out, topk_gate_out, group_counts_out, ws,
                                   MOGE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t moge_w8_weights_size(const moge_dims_t* dims) {
  const std::string saved = g_last_error;
  const moge_status_t s = check_w8_dims(dims);
  g_last_error = saved;
  if (s != MOGE_OK) return 0;
  return moge::w8_parts(dims->d, dims->N, dims->inter, dims->shared_inter).total;
}

moge_status_t moge_pack_weights_w8(const moge_dims_t* dims, const int8_t* q_gate,
                                   const int8_t* q_up, const int8_t* q_down, const float* s_gate,
                                   const float* s_up, const float* s_down, const int8_t* qs_gate,
                                   const int8_t* qs_up, const int8_t* qs_down,
                                   const float* ss_gate, const float* ss_up,
                                   const float* ss_down, void* w8, size_t w8_bytes,
                                   void* stream) {
  CHECK(check_w8_dims(dims));
  const bool shared = dims->shared_inter > 0;
  CHECK(check_ptr(q_gate, 16, "q_gate", true));
  CHECK(check_ptr(q_up, 16, "q_up", true));
  CHECK(check_ptr(q_down, 16, "q_down", true));
  CHECK(check_ptr(s_gate, 4, "s_gate", true));
  CHECK(check_ptr(s_up, 4, "s_up", true));
  CHECK(check_ptr(s_down, 4, "s_down", true));
  CHECK(check_ptr(qs_gate, 16, "qs_gate", shared));
  CHECK(check_ptr(qs_up, 16, "qs_up", shared));
  CHECK(check_ptr(qs_down, 16, "qs_down", shared));
  CHECK(check_ptr(ss_gate, 4, "ss_gate", shared));
  CHECK(check_ptr(ss_up, 4, "ss_up", shared));
  CHECK(check_ptr(ss_down, 4, "ss_down", shared));
  CHECK(check_ptr(w8, 256, "w8", true));
  const int d = dims->d, N = dims->N, I = dims->inter, Is = dims->shared_inter;
  const moge::W8Parts wp = moge::w8_parts(d, N, I, Is);
  if (w8_bytes < wp.total)
    return fail(MOGE_ERR_INVALID_ARG, "w8 buffer has %zu bytes, need %zu", w8_bytes, wp.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int8_t* dst = static_cast<int8_t*>(w8);
  auto copy = [&](size_t off, const float* src, size_t n, const char* what) {
    return hip_check(hipMemcpyAsync(dst + off, src, n * 4, hipMemcpyDeviceToDevice, st), what);
  };
  CHECK(hip_check(moge::launch_w8_pack(q_gate, q_up, N, I, d, dst + wp.routed_gu, st),
                  "pack int8 routed gate/up"));
  CHECK(hip_check(moge::launch_w8_pack(q_down, nullptr, N, d, I, dst + wp.routed_down, st),
                  "pack int8 routed down"));
  CHECK(copy(wp.s_gate, s_gate, (size_t)N * I, "copy gate scales"));
  CHECK(copy(wp.s_up, s_up, (size_t)N * I, "copy up scales"));
  CHECK(copy(wp.s_down, s_down, (size_t)N * d, "copy down scales"));
  if (shared) {
    CHECK(hip_check(moge::launch_w8_pack(qs_gate, qs_up, 1, Is, d, dst + wp.shared_gu, st),
                    "pack int8 shared gate/up"));
    CHECK(hip_check(moge::launch_w8_pack(qs_down, nullptr, 1, d, Is, dst + wp.shared_down, st),
                    "pack int8 shared down"));
    CHECK(copy(wp.ss_gate, ss_gate, (size_t)Is, "copy shared gate scales"));
    CHECK(copy(wp.ss_up, ss_up, (size_t)Is, "copy shared up scales"));
    CHECK(copy(wp.ss_down, ss_down, (size_t)d, "copy shared down scales"));
  }
  return ok();
}

moge_status_t moge_quantize_weights_w8(const moge_dims_t* dims, const void* w_gate,
                                       const void* w_up, const void* w_down, const void* ws_gate,
                                       const void* ws_up, const void* ws_down, void* w8,
                                       size_t w8_bytes, void* stream) {
  CHECK(check_w8_dims(dims));
  const bool shared = dims->shared_inter > 0;
  CHECK(check_ptr(w_gate, 16, "w_gate", true));
  CHECK(check_ptr(w_up, 16, "w_up", true));
  CHECK(check_ptr(w_down, 16, "w_down", true));
  CHECK(check_ptr(ws_gate, 16, "ws_gate", shared));
  CHECK(check_ptr(ws_up, 16, "ws_up", shared));
  CHECK(check_ptr(ws_down, 16, "ws_down", shared));
  CHECK(check_ptr(w8, 256, "w8", true));
  const int d = dims->d, N = dims->N, I = dims->inter, Is = dims->shared_inter;
  const moge::W8Parts wp = moge::w8_parts(d, N, I, Is);
  if (w8_bytes < wp.total)
    return fail(MOGE_ERR_INVALID_ARG, "w8 buffer has %zu bytes, need %zu", w8_bytes, wp.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(w8);
  int8_t* dst = reinterpret_cast<int8_t*>(base);
  auto sc = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  CHECK(hip_check(moge::launch_w8_quantize(w_gate, w_up, N, I, d, dst + wp.routed_gu,
                                           sc(wp.s_gate), sc(wp.s_up), st),
                  "quantize routed gate/up"));
  CHECK(hip_check(moge::launch_w8_quantize(w_down, nullptr, N, d, I, dst + wp.routed_down,
                                           sc(wp.s_down), nullptr, st),
                  "quantize routed down"));
  if (shared) {
    CHECK(hip_check(moge::launch_w8_quantize(ws_gate, ws_up, 1, Is, d, dst + wp.shared_gu,
                                             sc(wp.ss_gate), sc(wp.ss_up), st),
                    "quantize shared gate/up"));
    CHECK(hip_check(moge::launch_w8_quantize(ws_down, nullptr, 1, d, Is, dst + wp.shared_down,
                                             sc(wp.ss_down), nullptr, st),
                    "quantize shared down"));
  }
  return ok();
}

moge_status_t moge_layer_forward_w8(const moge_dims_t* dims, const void* x, const void* w_router,
                                    const float* router_bias, const void* w8,
                                    const float* logits_in, void* y, float* logits_out,
                                    int32_t* topk_idx_out, float* topk_gate_out,
                                    int32_t* group_counts_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  CHECK(check_w8_dims(dims));
  CHECK(check_ptr(w8, 256, "w8", true));
  const moge::W8Parts wp = moge::w8_parts(dims->d, dims->N, dims->inter, dims->shared_inter);
  const char* base = static_cast<const char*>(w8);
  auto sc = [&](size_t off) { return reinterpret_cast<const float*>(base + off); };
  Weights w;
  w.w8 = true;
  w.p_gu = base + wp.routed_gu;
  w.p_down = base + wp.routed_down;
  w.sc_gate = sc(wp.s_gate);
  w.sc_up = sc(wp.s_up);
  w.sc_down = sc(wp.s_down);
  if (dims->shared_inter > 0) {
    w.ps_gu = base + wp.shared_gu;
    w.ps_down = base + wp.shared_down;
    w.ssc_gate = sc(wp.ss_gate);
    w.ssc_up = sc(wp.ss_up);
    w.ssc_down = sc(wp.ss_down);
  }
  return layer_impl(dims, x, w_router, router_bias, w, logits_in, y, logits_out, topk_idx_out,
                    topk_gate_out, group_counts_out, ws, ws_bytes, stream);
}

}  // extern "C"
