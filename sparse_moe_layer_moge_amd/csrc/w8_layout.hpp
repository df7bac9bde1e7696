// Weight-only int8 (W8A16) expert-weight buffer: int8 codes in MFMA fragment
// order plus one float32 scale per output channel (weight = scale * code).
//
// Code tile = 16 rows x 64 contraction elements = 1 KiB, stored as 64 chunks of 16
// consecutive contraction elements; chunk l holds row l % 16, elements
// 16*(l/16) .. 16*(l/16)+15 of the tile's 64.  One 16-byte lane load is then the A
// operand of two 16x16x32 MFMA steps (elements 0..7 and 8..15 of the chunk).
//
// Gate/up part of one expert (I rows of W_gate and of W_up, contraction d): for row
// block b < I/16 and step s < d/64, the gate tile then the up tile of rows
// 16b..16b+15 at tile index (b*(d/64) + s)*2 + {0, 1}.
// Down part of one expert (d rows, contraction I): for row block b < d/32 and step
// s < I/64, the tiles of rows 32b..32b+15 and 32b+16..32b+31 at tile index
// (b*(I/64) + s)*2 + {0, 1}.
// Buffer regions, each starting at a 256-byte boundary:
//   codes:  routed gate/up (experts 0..N-1), routed down, shared gate/up, shared down
//   scales: gate [N,I], up [N,I], down [N,d], shared gate [I_s], shared up [I_s],
//           shared down [d]          (shared parts absent when I_s = 0)
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moge {

constexpr int kW8Step = 64;          // contraction elements per code tile
constexpr int kW8TileBytes = 1024;   // 16 rows x 64 codes

struct W8Parts {
  size_t routed_gu, routed_down, shared_gu, shared_down;  // code regions
  size_t s_gate, s_up, s_down, ss_gate, ss_up, ss_down;   // scale regions
  size_t total;
  size_t gu_expert, down_expert;  // code bytes of one routed expert's parts
};

inline size_t w8_align(size_t v) { return (v + 255) & ~size_t(255); }

inline W8Parts w8_parts(int d, int N, int I, int Is) {
  W8Parts p;
  p.gu_expert = (size_t)2 * I * d;
  p.down_expert = (size_t)d * I;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += w8_align(bytes);
    return at;
  };
  p.routed_gu = take((size_t)N * p.gu_expert);
  p.routed_down = take((size_t)N * p.down_expert);
  p.shared_gu = take((size_t)2 * Is * d);
  p.shared_down = take((size_t)d * Is);
  p.s_gate = take((size_t)N * I * 4);
  p.s_up = take((size_t)N * I * 4);
  p.s_down = take((size_t)N * d * 4);
  p.ss_gate = take((size_t)Is * 4);
  p.ss_up = take((size_t)Is * 4);
  p.ss_down = take(Is > 0 ? (size_t)d * 4 : 0);
  p.total = o;
  return p;
}

}  // namespace moge
