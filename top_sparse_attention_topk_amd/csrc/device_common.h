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
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
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
