// Device helpers shared by the GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define DG_LDS __attribute__((address_space(3)))
// read-only global data addressed uniformly: loads go through the scalar cache
#define DG_CONST __attribute__((address_space(4)))

// 16-byte chunk swizzle inside a 128-byte LDS row: the 16 rows one MFMA
// operand read touches at the same logical chunk land on distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> a packed bf16 pair (a in the low half), rounded to nearest
// even by the gfx950 conversion instruction (v_cvt_pk_bf16_f32, under the
// default round-to-nearest-even mode); NaN stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

// s_waitcnt immediate that waits for vmcnt <= n and leaves the other counters alone
// (gfx9 layout: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned (used
// before a barrier after which other waves overwrite the slot it read).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Map a workgroup id to a linear tile id so that the tiles one XCD runs are a
// contiguous range: workgroups are dealt to the 8 XCDs round-robin, and XCD x
// is given tiles [start_x, start_x + count_x).
__device__ __forceinline__ int xcd_tile(int bid, int tiles) {
  const int x = bid & 7;
  const int local = bid >> 3;
  const int q = tiles >> 3;
  const int r = tiles & 7;
  return x * q + (x < r ? x : r) + local;
}

// Tile id of round s of a walk over `tiles` tiles by `g` persistent
// workgroups in lockstep rounds: round s covers ids [s g, s g + g), and inside
// a round each XCD takes a contiguous run, so at any time all XCDs work on
// neighbouring tiles (the grouped forms: the same few experts' weights, shared
// through the Infinity Cache).
__device__ __forceinline__ int round_tile(int bid, int s, int g, int tiles) {
  const int left = tiles - s * g;
  return s * g + xcd_tile(bid, left < g ? left : g);
}

// Linear tile id -> (m, n) with groups of gm m-tiles walked column by column,
// so concurrently running tiles share operand rows in L2.
__device__ __forceinline__ void grouped_mn(int t, int m_tiles, int n_tiles, int gm, int* m, int* n) {
  const int per_group = gm * n_tiles;
  const int g = t / per_group;
  const int first_m = g * gm;
  const int gsz = (m_tiles - first_m) < gm ? (m_tiles - first_m) : gm;
  const int in = t - g * per_group;
  *m = first_m + in % gsz;
  *n = in / gsz;
}

}  // namespace dg
