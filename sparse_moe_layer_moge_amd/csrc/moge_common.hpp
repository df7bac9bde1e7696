// Device-side helpers shared by the MoGE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moge {

constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Buffer resources: a base address and a byte range held in scalar registers.
// A buffer load takes a 32-bit per-lane offset plus a wave-uniform scalar offset,
// so a streaming loop needs no 64-bit address registers per in-flight load, and
// loads outside the range return zeros instead of faulting.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferConfigGfx9 = 0x00020000;  // raw (untyped) buffer, gfx9 family
constexpr int kLoadNonTemporal = 2;            // cache-policy bit: streamed once

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                           kBufferConfigGfx9);
}

// ---------------------------------------------------------------------------
// Eight consecutive elements along the contraction dimension: the per-lane share
// of one K=32 step of a 16x16 MFMA tile.  bf16: 16 bytes, one v_mfma 16x16x32.
// float: 32 bytes, eight v_mfma 16x16x4 (element j of every lane feeds the j-th
// instruction; A and B use the same element->k assignment, so the sum over the 32
// k values is complete whatever the order).
// ---------------------------------------------------------------------------
template <typename E> struct Frag8;

template <> struct Frag8<bf16> {
  u32x4 v;
  template <int AUX>
  __device__ __forceinline__ void load_buf(Rsrc r, uint32_t voff, uint32_t soff) {
    v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
  }
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load_nt(const bf16* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
};

template <> struct Frag8<float> {
  f32x4 lo, hi;
  template <int AUX>
  __device__ __forceinline__ void load_buf(Rsrc r, uint32_t voff, uint32_t soff) {
    lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
    hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, AUX));
  }
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4*>(p);
    hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ void zero() {
    lo = f32x4{0.f, 0.f, 0.f, 0.f};
    hi = lo;
  }
};

// acc[16x16] += A[16x32] * B[32x16]; lane l supplies row (l%16) of A and column
// (l%16) of B, k-elements 8*(l/16)..8*(l/16)+7.  Result: lane l, register i holds
// D[4*(l/16)+i][l%16].
__device__ __forceinline__ f32x4 mfma_step(const Frag8<bf16>& a, const Frag8<bf16>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                 __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_step(const Frag8<float>& a, const Frag8<float>& b, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename E> __device__ __forceinline__ E from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// store four consecutive results (16 B float, 8 B bf16)
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 b;
  b[0] = static_cast<bf16>(v[0]);
  b[1] = static_cast<bf16>(v[1]);
  b[2] = static_cast<bf16>(v[2]);
  b[3] = static_cast<bf16>(v[3]);
  *reinterpret_cast<bf16x4*>(p) = b;
}

// silu(a) = a * sigmoid(a), the reciprocal by v_rcp_f32 (about 1 ulp) rather than an
// IEEE division, whose ten-instruction sequence per value made most of the
// epilogue of a 256-row gate/up tile (96 values per lane); the result is rounded
// to bf16 (or summed in float32 to 2^-23 relative) either way
__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// ---------------------------------------------------------------------------
// wave reductions (fixed butterfly order: deterministic)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum of an int over the 64 lanes with DPP moves, which stay in
// the vector unit (a shuffle is an LDS permute with a round trip each): shifts by
// 1, 2, 4 and 8 lanes inside every row of 16 lanes, then lane 15 added to row 1
// and 3 and lane 31 to rows 2 and 3.  Lanes with no source lane add 0.
__device__ __forceinline__ int wave_scan_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}
// lane `src` (wave-uniform) of v
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = threadIdx.x & (kWave - 1);
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moge
