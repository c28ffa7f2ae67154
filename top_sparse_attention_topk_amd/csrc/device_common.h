// Device helpers shared by the gfx950 kernels of libtka (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tka {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// Order-preserving key of an fp32 score: larger key <=> ranks higher.
// -0 and +0 share one key; every NaN maps to key 0, below -inf (0x007fffff).
// Integer selects only (no branch): negative scores flip every bit, the rest
// set the sign bit.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t z = u == 0x80000000u ? 0u : u;
  const uint32_t key = z ^ ((uint32_t)((int32_t)z >> 31) | 0x80000000u);
  return (u & 0x7fffffffu) > 0x7f800000u ? 0u : key;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bytes of a row as floats: 8 bf16 values or 4 fp32 values.
template <bool BF16>
struct Unpack;
template <>
struct Unpack<true> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void run(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
};
template <>
struct Unpack<false> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void run(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
// streaming (non-temporal) 16-byte load for data read exactly once
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int count_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// LDS written by some lanes of a wave, read by others: wait for this wave's LDS writes
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
}

// gfx950 lane swaps between 16-lane rows (v_permlane16_swap: x[0] holds rows 0,0,2,2 and x[1]
// rows 1,1,3,3 of v) and between wave halves (v_permlane32_swap: x[0] holds the low half twice,
// x[1] the high half). Plain VALU moves, no LDS crossbar.
__device__ __forceinline__ void rows_swap16(uint32_t v, uint32_t& even, uint32_t& odd) {
  const auto x = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  even = x[0];
  odd = x[1];
}
__device__ __forceinline__ void halves_swap32(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto x = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = x[0];
  hi = x[1];
}
// v + v of lane l ^ 16 and v + v of lane l ^ 32 (the same bits: the two terms commute)
__device__ __forceinline__ float sum_xor16(float v) {
  uint32_t e, o;
  rows_swap16(__float_as_uint(v), e, o);
  return __uint_as_float(e) + __uint_as_float(o);
}
__device__ __forceinline__ float sum_xor32(float v) {
  uint32_t lo, hi;
  halves_swap32(__float_as_uint(v), lo, hi);
  return __uint_as_float(lo) + __uint_as_float(hi);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// v of another lane through a DPP pattern (every lane active; patterns within a 16-lane row)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of W lanes (W = 2 .. 64, a power of two), the total in every lane of
// the group. Each step adds a lane that holds the same partial as the xor-butterfly partner (xor
// 1 and 2 by quad permutes, then the half-row and row mirrors, then row and half swaps), so the
// result has the bits of the xor butterfly: a + b == b + a.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W: a power of two up to 64");
  if constexpr (W >= 2) v += dpp_mov<0xb1>(v);   // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_mov<0x4e>(v);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v += dpp_mov<0x140>(v); // row_mirror
  if constexpr (W >= 32) v = sum_xor16(v);
  if constexpr (W >= 64) v = sum_xor32(v);
  return v;
}

// Sums (and maxima) over the lanes l ^ O, l ^ 2O, ..., l ^ 32 (groups of O lanes merged
// position by position, O = 8, 16 or 32): exact xor partners, by row rotation for 8 and by the
// row and half swaps for 16 and 32; the bits of the xor butterfly.
template <int O>
__device__ __forceinline__ float cross_sum(float v) {
  static_assert(O == 8 || O == 16 || O == 32 || O == 64, "O: 8, 16, 32 (64: nothing to merge)");
  if constexpr (O <= 8) v += dpp_mov<0x128>(v);  // row_ror:8 = lane ^ 8 within the row
  if constexpr (O <= 16) v = sum_xor16(v);
  if constexpr (O <= 32) v = sum_xor32(v);
  return v;
}
template <int O>
__device__ __forceinline__ float cross_max(float v) {
  static_assert(O == 8 || O == 16 || O == 32 || O == 64, "O: 8, 16, 32 (64: nothing to merge)");
  if constexpr (O <= 8) v = fmaxf(v, dpp_mov<0x128>(v));
  if constexpr (O <= 16) {
    uint32_t e, o;
    rows_swap16(__float_as_uint(v), e, o);
    v = fmaxf(__uint_as_float(e), __uint_as_float(o));
  }
  if constexpr (O <= 32) {
    uint32_t lo, hi;
    halves_swap32(__float_as_uint(v), lo, hi);
    v = fmaxf(__uint_as_float(lo), __uint_as_float(hi));
  }
  return v;
}

// maximum across the 64 lanes (every lane active)
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xb1>(v));
  v = fmaxf(v, dpp_mov<0x4e>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return cross_max<16>(v);
}

// Inclusive prefix sum across the 64 lanes, on DPP lane moves (no LDS crossbar): Kogge-Stone
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes (lanes shifted in from outside the row add
// 0), then row 15's total is broadcast into rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return v;
}

// Minimum across the 64 lanes, as wave_max_u32 below.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = min(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}

// Maximum across the 64 lanes (wave-uniform result): DPP swaps inside quads, half rows and rows
// leave each row's maximum in all its lanes; the four rows are then read from lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Workgroups are dispatched to the 8 XCDs (each with its own L2) in turn by
// their linear id. This bijection on [0, total) gives consecutive logical ids
// to the workgroups of one XCD, in their dispatch order, so that work sharing
// data (the query heads of one KV group) shares an L2.
constexpr unsigned kXcds = 8;
__device__ __forceinline__ unsigned xcd_logical_id(unsigned hid, unsigned total) {
  const unsigned xcd = hid % kXcds, i = hid / kXcds, q = total / kXcds, r = total % kXcds;
  return xcd < r ? xcd * (q + 1) + i : r * (q + 1) + (xcd - r) * q + i;
}

}  // namespace tka
