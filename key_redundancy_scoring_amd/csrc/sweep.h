// Building blocks shared by the Gram sweeps (gram.hip: the repair pass's
// restricted sweep; tri.hip: the single-order score sweep): launch shapes,
// LDS stage buffers filled by direct global->LDS loads, the XOR swizzle of
// the MFMA A-operand reads, the accumulator layout of
// v_mfma_f32_32x32x16_bf16 and exact fp64 dot products of bf16 chunks.
#pragma once

#include "internal.h"

#define TWINKV_LDS __attribute__((address_space(3)))
#define TWINKV_GLOBAL __attribute__((address_space(1)))
#define TWINKV_INLINE __attribute__((always_inline))

namespace twinkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Launch shape of the sweep: head dim, row blocks of 32 per wave, waves per
// workgroup, columns per LDS stage, and waves per SIMD the registers are
// budgeted for (two stage buffers of SC columns per workgroup must fit the
// CU's LDS that many times over).
template <int D_, int RB_, int WAVES_, int SC_, int OCC_>
struct GramShape {
  static constexpr int D = D_, RB = RB_, WAVES = WAVES_, SC = SC_, OCC = OCC_;
  static constexpr int ROWS = WAVES * RB * 32;
};
// vmcnt(0), other counters untouched (gfx9 s_waitcnt encoding)
constexpr unsigned kWaitVm0 = 0x0F70;

// One stage buffer: column keys (swizzled 16-byte chunks), inverse norms and
// positions (repair mode).
template <int D, int SC>
struct Stage {
  uint4 keys[SC * (D / 8)];
  float rinv[SC];
  int32_t pos[SC];
};

// A stage buffer of the score sweep: column keys and inverse norms only
// (the columns are the head's own positions).
template <int D, int SC>
struct StageK {
  uint4 keys[SC * (D / 8)];
  float rinv[SC];
};

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const TWINKV_GLOBAL void*)src, (TWINKV_LDS void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const TWINKV_GLOBAL void*)src, (TWINKV_LDS void*)lds_wave_base, 4, 0, 0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

__device__ __forceinline__ float max16(const float* y) {
  const float m01 = max3f(y[0], y[1], y[2]);
  const float m02 = max3f(y[3], y[4], y[5]);
  const float m03 = max3f(y[6], y[7], y[8]);
  const float m04 = max3f(y[9], y[10], y[11]);
  const float m05 = max3f(y[12], y[13], y[14]);
  const float m11 = max3f(m01, m02, m03);
  const float m12 = max3f(m04, m05, y[15]);
  return __builtin_fmaxf(m11, m12);
}

__device__ __forceinline__ double dot8_exact(uint4 a, uint4 b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
  double s = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s += (double)(__uint_as_float(x[t] << 16) * __uint_as_float(y[t] << 16));
    s += (double)(__uint_as_float(x[t] & 0xffff0000u) * __uint_as_float(y[t] & 0xffff0000u));
  }
  return s;
}

// (exact cosine, position) -> one 64-bit key whose unsigned order is the
// cosine's, then the lower position; 0 is below every key.  The low bits
// selected by idx_mask (2^b - 1 with 2^b >= N) carry idx_mask - position in
// place of the cosine's lowest mantissa bits, so two cosines that differ only
// there (by less than 2^(b-52) relative) rank as equal and the lower position
// wins.
__device__ __forceinline__ uint64_t pack_best(double sim, int idx, uint64_t idx_mask) {
  uint64_t u = (uint64_t)__double_as_longlong(sim + 0.0);
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return (u & ~idx_mask) | (idx_mask - (uint64_t)idx);
}
__device__ __forceinline__ int unpack_idx(uint64_t u, uint64_t idx_mask) { return (int)(idx_mask - (u & idx_mask)); }

// XOR swizzle of the 16-byte chunks of stage column c (CH chunks per key).
// Chunk k of column c lives at slot c*CH + (k ^ swz(c)).  For the A-operand
// reads (lane l reads chunk k of column l mod 32) this puts any 8 consecutive
// lanes on distinct 16-byte bank groups of a 128-byte row and any 16 on
// distinct groups of a 256-byte row.  It repeats every kSwzPeriod columns, so
// the per-lane part of an address is the same for every 32-column tile.
constexpr int kSwzPeriod = 16;
template <int CH>
__device__ __forceinline__ int swz(int c) {
  return CH == 8 ? ((c ^ ((c >> 3) & 1)) & 7) : (c & 15);
}

// column offset (within a 32-column tile) of accumulator r in half-wave h
__device__ __forceinline__ int tile_col(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace
}  // namespace twinkv
