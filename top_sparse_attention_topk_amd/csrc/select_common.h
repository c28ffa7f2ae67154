// Exact selection building blocks shared by the select kernels and the
// gather's in-workgroup row select. Order: i before j when s_i > s_j, or
// s_i == s_j and i < j (-0 == +0, NaN below every number), through the
// order-preserving 32-bit score keys.
#pragma once

#include "device_common.h"

namespace tka {

constexpr int ST = 256;  // threads per workgroup
constexpr int SW = 4;    // waves per workgroup
constexpr int NB0 = 4096;

// LDS of a select workgroup of NW waves (at most 16: one scan slot per wave)
template <int NB, int NW = SW>
struct alignas(16) SelSmemT {
  static_assert(NW >= 1 && NW <= 16, "at most 16 waves");
  static constexpr int kBins = NB;
  static constexpr int kWaves = NW;
  uint32_t hist[NB];
  uint32_t scan[16];
  uint32_t res[2];
  uint32_t aux;
  uint32_t cnt[NW];
  uint32_t gt[NW], eq[NW];
  uint32_t obase[NW], eqbase[NW];
};
using SelSmem = SelSmemT<NB0>;

// Inclusive scan over the workgroup (NW waves). TRAIL = false leaves out the closing barrier
// that lets sm.scan be written again: for callers that pass another barrier first.
template <int NW, typename SM, bool TRAIL = true>
__device__ uint32_t block_incl_scan_t(uint32_t v, SM& sm, uint32_t* total) {
  const int w = threadIdx.x >> 6, l = lane_id();
  uint32_t x = wave_incl_scan(v);
  if (l == 63) sm.scan[w] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    off += (i < w) ? sm.scan[i] : 0u;
    tot += sm.scan[i];
  }
  if (TRAIL) __syncthreads();
  *total = tot;
  return x + off;
}

// Bin b with above(b) < need <= above(b) + hist[b], above(b) = sum of the
// bins over b. Result in sm.res (bin, above). need must not exceed the total.
template <int NW, typename SM>
__device__ void find_bin_t(const uint32_t* hist, int nb, uint32_t need, SM& sm) {
  const int t = threadIdx.x;
  const int per = nb / (64 * NW);
  uint32_t s = 0;
  for (int i = 0; i < per; ++i) s += hist[t * per + i];
  uint32_t tot;
  const uint32_t incl = block_incl_scan_t<NW, SM, false>(s, sm, &tot);  // the barrier below closes it
  const uint32_t above = tot - incl;
  if (above < need && need <= above + s) {
    uint32_t acc = above;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t h = hist[t * per + i];
      if (acc + h >= need) {
        sm.res[0] = (uint32_t)(t * per + i);
        sm.res[1] = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

constexpr uint32_t RK_STASH = 256;  // a critical bin this small is ranked element by element

// The kk-th largest key (1 <= kk <= nvalid) among elements held PER per thread in registers
// (element e = threadIdx.x * PER + i; e >= nvalid ignored), and how many keys equal to it the
// select order keeps (the first ones by index). Histograms of SM::kBins bins over the keys' own range,
// each level narrowing to the bin that holds the kk-th key, until that bin is one key wide or holds
// at most RK_STASH keys, which are then ranked one by one. All threads call it.
template <int PER, typename SM>
__device__ __forceinline__ void block_kth_regs(const uint32_t (&key)[PER], int nvalid, uint32_t kk, SM& sm, uint32_t* T_out,
                               uint32_t* need_eq_out) {
  const int t = threadIdx.x, w = t >> 6, lane = lane_id();
  const int e0 = t * PER;
  constexpr int NB = SM::kBins;
  constexpr int NW = SM::kWaves, NT = 64 * NW;  // the workgroup: NW waves
  constexpr int LB = NB == 4096 ? 12 : (NB == 2048 ? 11 : (NB == 1024 ? 10 : 8));  // bits per level
  static_assert(NB == (1 << LB) && NB % NT == 0, "bins: 256, 1024, 2048 or 4096, a multiple of the threads");
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (e0 + i < nvalid) {
      mn = min(mn, key[i]);
      mx = max(mx, key[i]);
    }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane == 0) {
    sm.gt[w] = mn;
    sm.eq[w] = mx;
  }
  for (int i = t; i < NB; i += NT) sm.hist[i] = 0;
  __syncthreads();
  uint32_t base = sm.gt[0], hi = sm.eq[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    base = min(base, sm.gt[i]);
    hi = max(hi, sm.eq[i]);
  }
  const uint32_t span = hi - base;
  int sh = span >= (uint32_t)NB ? (32 - __clz(span)) - LB : 0;  // span >> sh < NB
  uint32_t width = span;  // keys of the current range: [base, base + width]
  uint32_t need = kk;
  for (;;) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (e0 + i < nvalid && key[i] >= base && key[i] - base <= width) atomicAdd(&sm.hist[(key[i] - base) >> sh], 1u);
    __syncthreads();
    find_bin_t<NW>(sm.hist, NB, need, sm);
    const uint32_t bin = sm.res[0], above = sm.res[1], inbin = sm.hist[bin];
    __syncthreads();  // every thread has read the histogram
    need -= above;
    base += bin << sh;
    if (sh == 0) {  // the bin is one key
      *T_out = base;
      *need_eq_out = need;
      return;
    }
    width = (1u << sh) - 1u;
    if (inbin <= RK_STASH) {
      if (t == 0) sm.aux = 0u;
      __syncthreads();
      uint32_t* stash = sm.hist;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (e0 + i < nvalid && key[i] >= base && key[i] - base <= width) stash[atomicAdd(&sm.aux, 1u)] = key[i];
      __syncthreads();
      for (uint32_t j = t; j < inbin; j += NT) {
        const uint32_t v = stash[j];
        uint32_t gt = 0, ge = 0;
        for (uint32_t x = 0; x < inbin; ++x) {
          const uint32_t y = stash[x];
          gt += y > v;
          ge += y >= v;
        }
        if (gt < need && need <= ge) {  // v is the need-th largest of the bin (all such j agree)
          sm.res[0] = v;
          sm.res[1] = need - gt;
        }
      }
      __syncthreads();
      *T_out = sm.res[0];
      *need_eq_out = sm.res[1];
      return;
    }
    sh = sh >= LB ? sh - LB : 0;  // the next level's NB bins cover the bin's 2^sh_old keys
    for (int i = t; i < NB; i += NT) sm.hist[i] = 0;
    __syncthreads();
  }
}

// As block_emit_regs below, but the kept (position, score bits) go to their slots in LDS first
// (lidx, lsel: at least kk entries each) and out with 16-byte stores in slot order, so that the
// global writes are whole lines rather than one scattered word per lane. kk: the number kept.
template <int PER, typename BitsOf, typename PosOf, typename SM>
__device__ __forceinline__ void block_emit_regs_staged(const uint32_t (&key)[PER], BitsOf bits_of,
                                                       PosOf pos_of, int nvalid, uint32_t T, uint32_t need_eq,
                                                       int kk, SM& sm, uint32_t* lidx, uint32_t* lsel,
                                                       int32_t* __restrict__ oidx, float* __restrict__ osel) {
  const int e0 = threadIdx.x * PER;
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (e0 + i < nvalid) {
      ngt += key[i] > T;
      neq += key[i] == T;
    }
  const uint32_t v = (ngt << 16) | neq;  // totals stay below 2^16
  uint32_t tot;
  const uint32_t ex = block_incl_scan_t<SM::kWaves>(v, sm, &tot) - v;
  const uint32_t eqb = ex & 0xffffu;
  uint32_t slot = (ex >> 16) + min(eqb, need_eq), eqs = eqb;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (e0 + i >= nvalid) continue;
    bool take = key[i] > T;
    if (key[i] == T) take = eqs++ < need_eq;
    if (take) {
      lidx[slot] = (uint32_t)pos_of(i);
      lsel[slot] = bits_of(i);
      ++slot;
    }
  }
  __syncthreads();
  const bool vec = ((reinterpret_cast<uintptr_t>(oidx) | reinterpret_cast<uintptr_t>(osel)) & 15) == 0;
  for (int i = 4 * (int)threadIdx.x; i < kk; i += 4 * 64 * SM::kWaves) {
    if (vec && i + 3 < kk) {
      *reinterpret_cast<uint4*>(oidx + i) = *reinterpret_cast<const uint4*>(lidx + i);
      if (osel) *reinterpret_cast<uint4*>(osel + i) = *reinterpret_cast<const uint4*>(lsel + i);
    } else {
      for (int c = i; c < min(i + 4, kk); ++c) {
        oidx[c] = (int32_t)lidx[c];
        if (osel) osel[c] = __uint_as_float(lsel[c]);
      }
    }
  }
}

// Emit, in index order, the elements with key > T and the first need_eq with key == T: their
// positions to oidx and score bits (bits_of(i) of the thread's element i) to osel (when given).
// One packed (greater, equal) block scan.
template <int PER, typename BitsOf, typename PosOf, typename SM>
__device__ __forceinline__ void block_emit_regs(const uint32_t (&key)[PER], BitsOf bits_of, PosOf pos_of, int nvalid,
                                uint32_t T, uint32_t need_eq, SM& sm, int32_t* __restrict__ oidx,
                                float* __restrict__ osel) {
  const int e0 = threadIdx.x * PER;
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (e0 + i < nvalid) {
      ngt += key[i] > T;
      neq += key[i] == T;
    }
  const uint32_t v = (ngt << 16) | neq;  // totals stay below 2^16
  uint32_t tot;
  const uint32_t ex = block_incl_scan_t<SM::kWaves>(v, sm, &tot) - v;
  const uint32_t eqb = ex & 0xffffu;
  uint32_t slot = (ex >> 16) + min(eqb, need_eq), eqs = eqb;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (e0 + i >= nvalid) continue;
    bool take = key[i] > T;
    if (key[i] == T) take = eqs++ < need_eq;
    if (take) {
      oidx[slot] = pos_of(i);
      if (osel) osel[slot] = __uint_as_float(bits_of(i));
      ++slot;
    }
  }
}


}  // namespace tka
