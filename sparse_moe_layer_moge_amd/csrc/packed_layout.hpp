// Packed expert-weight layout (MFMA fragment order), used by the weight-streaming
// and tile kernels and written by moge_pack_weights.
//
// A fragment tile covers 16 weight rows x 32 contraction elements and is stored as
// 64 lane chunks of 8 consecutive contraction elements: chunk l holds row (l % 16),
// elements 8*(l / 16) .. 8*(l / 16) + 7 of the tile's 32.  Tile bytes = 512 * es.
//
// Gate/up part of one expert (I rows of W_gate and of W_up, contraction d): for
// row block b < I/16 and step s < d/32, the gate tile (rows 16b..16b+15) and then
// the up tile (same rows) at tile index (b * (d/32) + s) * 2 + {0, 1}.
// Down part of one expert (d rows of W_down, contraction I): for row block
// b < d/32 (32 rows) and step s < I/32, the tiles of rows 32b..32b+15 and
// 32b+16..32b+31 at tile index (b * (I/32) + s) * 2 + {0, 1}.
// Buffer: [routed gate/up, expert 0..N-1][routed down, expert 0..N-1]
//         [shared gate/up][shared down]   (shared parts absent when I_s = 0)
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moge {

struct PackedParts {
  size_t routed_gu, routed_down, shared_gu, shared_down, total;
  size_t gu_expert, down_expert;  // bytes of one routed expert's parts
};

inline PackedParts packed_parts(int d, int N, int I, int Is, int es) {
  PackedParts p;
  p.gu_expert = (size_t)2 * I * d * es;
  p.down_expert = (size_t)d * I * es;
  p.routed_gu = 0;
  p.routed_down = p.routed_gu + (size_t)N * p.gu_expert;
  p.shared_gu = p.routed_down + (size_t)N * p.down_expert;
  p.shared_down = p.shared_gu + (size_t)2 * Is * d * es;
  p.total = p.shared_down + (size_t)d * Is * es;
  return p;
}

constexpr int kTileElems = 512;  // 16 rows x 32 contraction elements

}  // namespace moge
