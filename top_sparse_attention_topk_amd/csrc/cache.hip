// Cache maintenance for one decode step, for gfx950.
//
// "Sparse Attention in LLM Inference", "Changes in Caching Strategy": the
// sparse layer reads its cache through a position index, so the caches keep
// one row per position, appended as tokens arrive. The proxy caches of
// "Sparse Attention Landscape" follow: MoBA's mean-pooled block keys ("Block
// Sparse Attention") and the lightning indexer's low-dimensional keys
// ("Token Sparse Attention"), stored here as OCP E4M3FN codes.
#include "device_common.h"
#include "internal.h"

namespace tka {

// One workgroup per (b, KV head): the new key and value rows (row_bytes each,
// a multiple of 16) go to position pos of the strided caches.
__global__ __launch_bounds__(64) void append_rows_kernel(const uint8_t* __restrict__ knew,
                                                         const uint8_t* __restrict__ vnew, uint8_t* __restrict__ K,
                                                         uint8_t* __restrict__ V, int Hkv, int row_bytes, int es,
                                                         int64_t sb, int64_t sh, int64_t sl, int pos) {
  const int task = blockIdx.x;
  const int b = task / Hkv, g = task % Hkv;
  const int64_t dst = ((int64_t)b * sb + (int64_t)g * sh + (int64_t)pos * sl) * es;
  const int64_t src = (int64_t)task * row_bytes;
  for (int i = threadIdx.x * 16; i < row_bytes; i += 64 * 16) {
    if (knew) *reinterpret_cast<uint4*>(K + dst + i) = *reinterpret_cast<const uint4*>(knew + src + i);
    if (vnew) *reinterpret_cast<uint4*>(V + dst + i) = *reinterpret_cast<const uint4*>(vnew + src + i);
  }
}

// fp32 -> OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// largest finite 448, S.1111.111 is NaN): round to nearest, ties to even,
// |x| >= 448 (infinities too) saturates to 448, NaN -> 0x7f, the sign kept.
// Below the least normal (2^-6) codes are multiples of 2^-9; above it the
// 23-bit fp32 mantissa is rounded to 3 bits.
__device__ __forceinline__ uint8_t e4m3_rne_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x != x) return 0x7f;
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);  // |x| >= 448
  if (a < 0x3c800000u) {                                   // |x| < 2^-6: code = |x| / 2^-9, rounded
    const uint32_t m = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);  // exact scaling; ties to even
    return (uint8_t)(sign | m);                            // m = 8 is the least normal, code 0x08
  }
  int e = (int)(a >> 23) - 127;  // -6 .. 8
  uint32_t keep = (a >> 20) & 7u;
  const uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0;
    ++e;
  }
  return (uint8_t)(sign | ((uint32_t)(e + 7) << 3) | keep);  // |x| < 448: at most 448 = 0x7e
}

// One workgroup per sequence: the new indexer key (d_I fp32) to row pos of kI [B, Lc, d_I].
__global__ __launch_bounds__(256) void append_indexer_kernel(const float* __restrict__ kI_new,
                                                             uint8_t* __restrict__ kI, int dI, int Lc, int pos) {
  const int b = blockIdx.x;
  for (int t = threadIdx.x; t < dI; t += 256) kI[((int64_t)b * Lc + pos) * dI + t] = e4m3_rne_sat(kI_new[b * dI + t]);
}

void launch_append_rows(const void* knew, const void* vnew, void* K, void* V, int B, int Hkv, int row_bytes, int es,
                        int64_t sb, int64_t sh, int64_t sl, int pos, hipStream_t st) {
  if (B <= 0 || Hkv <= 0) return;
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)(B * Hkv)), dim3(64), 0, st, (const uint8_t*)knew,
                     (const uint8_t*)vnew, (uint8_t*)K, (uint8_t*)V, Hkv, row_bytes, es, sb, sh, sl, pos);
}

void launch_append_indexer(const float* kI_new, uint8_t* kI, int B, int dI, int Lc, int pos, hipStream_t st) {
  if (B <= 0) return;
  hipLaunchKernelGGL(append_indexer_kernel, dim3((unsigned)B), dim3(256), 0, st, kI_new, kI, dI, Lc, pos);
}

}  // namespace tka
