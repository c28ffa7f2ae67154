// Lightning-indexer score core ("Sparse Attention Landscape", "Token Sparse
// Attention": I[b,i] = sum_j w[b,j] * max(0, <qI[b,j], kI[b,i]>)), shared by
// the scoring kernel and the fused indexer step's candidate kernel so that
// both produce the same bits.
//
// E4M3FN inputs, v_mfma_scale_f32_32x32x64_f8f6f4 (both formats E4M3, unit
// scales): A = 32 indexer heads x 64 dims (lane l: head l%32, dims
// 32*(l/32)+[0,32)), B = 64 dims x 32 positions (lane l: position l%32, same
// dims), C[head][pos]: lane l holds position l%32 for heads 8a + 4*(l/32) + c.
// ReLU and the weighted head sum stay in registers; lanes l and l^32 add
// their halves of the head sum (a lane swap between the wave halves), so
// both hold the position's score.
#pragma once

#include "device_common.h"

namespace tka {

// One wave's query side: NT tiles of 32 heads, DI/64 contraction steps.
template <int DI, int NT>
struct IndexerQuery {
  i32x8_t aq[NT][DI / 64];
  float wt[NT][16];
};

template <int DI, int NT>
__device__ __forceinline__ void indexer_load_query(IndexerQuery<DI, NT>& Q, const uint8_t* __restrict__ qI,
                                                   const float* __restrict__ w, int b, int HI, int lane) {
  constexpr int KS = DI / 64;
  const int j = lane & 31, half = lane >> 5;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int head = t * 32 + j;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
      if (head < HI) {
        const uint8_t* p = qI + ((int64_t)b * HI + head) * DI + 64 * s + 32 * half;
        lo = ld16(p);
        hi = ld16(p + 16);
      }
      i32x8_t v;
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
      Q.aq[t][s] = v;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int hh = t * 32 + 8 * a + 4 * half + c;
        Q.wt[t][4 * a + c] = hh < HI ? w[(int64_t)b * HI + hh] : 0.f;
      }
  }
}

// Scores of positions base + 32u + (lane & 31), u < UNR, into tot[u] (every
// lane; positions past L - 1 read row L - 1 and are to be ignored). kb: the
// sequence's key rows, DI bytes each.
template <int DI, int NT, int UNR>
__device__ __forceinline__ void indexer_round(const IndexerQuery<DI, NT>& Q, const uint8_t* __restrict__ kb, int base,
                                              int L, int lane, float (&tot)[UNR]) {
  constexpr int KS = DI / 64;
  const int j = lane & 31, half = lane >> 5;
  uint4 raw[UNR][KS][2];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int pos = min(base + 32 * u + j, L - 1);
    const uint8_t* row = kb + (int64_t)pos * DI + 32 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      raw[u][s][0] = ld16_stream(row + 64 * s);
      raw[u][s][1] = ld16_stream(row + 64 * s + 16);
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    float acc_tot = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        i32x8_t bk;
        bk[0] = raw[u][s][0].x; bk[1] = raw[u][s][0].y; bk[2] = raw[u][s][0].z; bk[3] = raw[u][s][0].w;
        bk[4] = raw[u][s][1].x; bk[5] = raw[u][s][1].y; bk[6] = raw[u][s][1].z; bk[7] = raw[u][s][1].w;
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Q.aq[t][s], bk, acc, 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_tot = fmaf(Q.wt[t][i], fmaxf(acc[i], 0.f), acc_tot);
    }
    tot[u] = sum_xor32(acc_tot);
  }
}

}  // namespace tka
