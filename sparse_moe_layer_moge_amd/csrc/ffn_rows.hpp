// Rows of one expert inside a streaming FFN segment (device side), shared by the
// bf16 and the weight-only int8 streaming kernels.
#pragma once

#include "moge_common.hpp"
#include "moge_internal.hpp"

namespace moge {

struct SegView {
  int lo, cnt;
};

// rows of expert e; offsets from the caller are clamped into [0, rows]; an expert
// with more rows than g.thr is left to the tile path (cnt = 0 here)
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
  if (v.cnt > g.thr) v.cnt = 0;
  return v;
}

}  // namespace moge
