// Exact top-k selection for gfx950 (TopK_j s_j of "Sparse Attention
// Landscape", "Block Sparse Attention"; the fixed budget of "Sparse Attention
// in LLM Inference", "The Significance of Top-K").
//
// Order: i before j when s_i > s_j, or s_i == s_j and i < j; -0 == +0; NaN
// below every number. Scores become order-preserving 32-bit keys and the
// k-th key T is found digit by digit (bits 31..20, 19..10, 9..0) with LDS
// histograms. Elements whose key is at least the lower edge of T's current
// digit range are compacted in position order (wave ballots + mbcnt), so the
// answer is emitted in ascending position with no sort: every key > T, and
// the first (k - #(key > T)) keys == T in position order.
//
// Two launch shapes:
//  - row mode: one workgroup per row (many rows). Pass 1 builds the level-0
//    histogram, pass 2 compacts the candidates into LDS; the rest runs on
//    LDS. Extra histogram passes (and a streaming emit) only when the
//    candidates do not fit (heavy ties).
//  - split mode: few long rows. Chunks of 4096 elements per workgroup build a
//    global histogram, then compact their candidates into per-chunk regions;
//    one workgroup per row finishes on the (small) candidate list.
#include <math.h>

#include <algorithm>
#include <cstddef>
#include <mutex>
#include <utility>
#include <vector>

#include "device_common.h"
#include "indexer_core.h"
#include "internal.h"
#include "select_common.h"

namespace tka {

constexpr int NB1 = 1024;
constexpr int UNR = 4;          // float4 loads per lane per round
constexpr int CHUNK = 4096;     // split mode: elements per workgroup
constexpr int SEL_SAMPLES = 2048;       // row mode: samples for the threshold of long rows
#ifndef TKA_SEL_SAMPLE_MIN_N
#define TKA_SEL_SAMPLE_MIN_N 16384
#endif
constexpr int SEL_SAMPLE_MIN_N = TKA_SEL_SAMPLE_MIN_N;  // shortest row that takes the sampled threshold
constexpr int SEL_SAMPLE_MAX_N = 262144;                // longest: a wave's segment fits 16-bit offsets
#ifndef TKA_SEL_U
#define TKA_SEL_U 16
#endif
constexpr int SEL_U = TKA_SEL_U;  // float4 loads per lane in flight in the sampled path's pass
constexpr int SUBCH = CHUNK / SW;

__device__ __forceinline__ int lv_shift(int lv) { return lv == 0 ? 20 : (lv == 1 ? 10 : 0); }
__device__ __forceinline__ int lv_bits(int lv) { return lv == 0 ? 12 : 10; }
__device__ __forceinline__ int lv_bins(int lv) { return lv == 0 ? NB0 : NB1; }
__device__ __forceinline__ uint32_t lv_digit(uint32_t key, int lv) {
  return (key >> lv_shift(lv)) & (lv == 0 ? 0xFFFu : 0x3FFu);
}
// the digits above level lv equal `prefix`
__device__ __forceinline__ bool lv_in_range(uint32_t key, int lv, uint32_t prefix) {
  return lv == 0 || (key >> lv_shift(lv - 1)) == prefix;
}

// A float whose score key is `key` (inverse of score_key up to -0 and NaN payloads).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ uint32_t block_incl_scan(uint32_t v, SelSmem& sm, uint32_t* total) {
  return block_incl_scan_t<SW>(v, sm, total);
}

__device__ void find_bin(const uint32_t* hist, int nb, uint32_t need, SelSmem& sm) {
  find_bin_t<SW>(hist, nb, need, sm);
}

__device__ __forceinline__ void load4(const float* s, int p, int end, bool aligned, float (&v)[4]) {
  if (aligned && p + 3 < end) {
    const float4 x = *reinterpret_cast<const float4*>(s + p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (p + j < end) ? s[p + j] : 0.f;
  }
}

// LDS histogram of digit lv over the elements of [r0, r1) inside the range.
__device__ void hist_pass(const float* s, int r0, int r1, bool aligned, int lv, uint32_t prefix, uint32_t* hist) {
  const int lane = lane_id();
  for (int base = r0; base < r1; base += 256 * UNR) {
    float v[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u) load4(s, base + u * 256 + 4 * lane, r1, aligned, v[u]);
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = base + u * 256 + 4 * lane + j;
        const uint32_t key = score_key(v[u][j]);
        if (p < r1 && lv_in_range(key, lv, prefix)) atomicAdd(&hist[lv_digit(key, lv)], 1u);
      }
  }
}

// Keys >= lo of [r0, r1), in position order, to cb/cp (first `cap` of them), U float4
// loads per lane in flight. Returns the number found (the same value in every lane).
template <int U>
__device__ uint32_t collect_pass_t(const float* s, int r0, int r1, bool aligned, uint32_t lo, uint32_t* cb,
                                   int32_t* cp, uint32_t cap) {
  const int lane = lane_id();
  uint32_t cnt = 0;
  for (int base = r0; base < r1; base += 256 * U) {
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) load4(s, base + u * 256 + 4 * lane, r1, aligned, v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bool f[4];
      uint32_t before = 0, tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = base + u * 256 + 4 * lane + j;
        f[j] = p < r1 && score_key(v[u][j]) >= lo;
        const uint64_t bl = ballot(f[j]);
        before += count_below(bl);
        tot += __popcll(bl);
      }
      uint32_t slot = cnt + before;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (f[j]) {
          if (slot < cap) {
            cb[slot] = __float_as_uint(v[u][j]);
            cp[slot] = base + u * 256 + 4 * lane + j;
          }
          ++slot;
        }
      }
      cnt += tot;
    }
  }
  return cnt;
}

__device__ uint32_t collect_pass(const float* s, int r0, int r1, bool aligned, uint32_t lo, uint32_t* cb,
                                 int32_t* cp, uint32_t cap) {
  return collect_pass_t<UNR>(s, r0, r1, aligned, lo, cb, cp, cap);
}

// collect_pass for a 16-byte aligned row whose segment ends are multiples of 4: every load is
// one float4 with no branch around it (past r1 the address is clamped to the last float4 of the
// segment and the values masked), so all U of a round are in flight together - a load under a
// condition makes the compiler wait for each one before the next.
template <int U>
__device__ __forceinline__ uint32_t collect_fast(const float* s, int r0, int r1, uint32_t lo, uint32_t* cb,
                                                 uint16_t* cp, uint32_t cap) {
  const int lane = lane_id();
  uint32_t cnt = 0;
  for (int base = r0; base < r1; base += 256 * U) {
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = *reinterpret_cast<const float4*>(s + min(base + u * 256 + 4 * lane, r1 - 4));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p0 = base + u * 256 + 4 * lane;
      const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      bool f[4];
      uint32_t before = 0, tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = p0 < r1 && score_key(v[j]) >= lo;
        const uint64_t bl = ballot(f[j]);
        before += count_below(bl);
        tot += __popcll(bl);
      }
      uint32_t slot = cnt + before;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (f[j]) {
          if (slot < cap) {
            cb[slot] = __float_as_uint(v[j]);
            cp[slot] = (uint16_t)(p0 + j - r0);  // offset in the segment: positions as 16 bits
          }
          ++slot;
        }
      }
      cnt += tot;
    }
  }
  return cnt;
}

// Radix search for the need-th largest key among the elements wave w owns
// ([0, cnt) through key_of(e)), through levels l0..2, starting from the
// digits `prefix` fixed above level l0. Returns T in sm.res[0] and the
// number of keys == T to keep in sm.res[1].
template <int NW, typename KeyOf>
__device__ void radix_kth_t(KeyOf key_of, uint32_t cnt, int l0, uint32_t prefix, uint32_t need, SelSmem& sm) {
  constexpr int U = 8;  // independent loads in flight per lane
  const int lane = lane_id();
  for (int l = l0; l <= 2; ++l) {
    const int nb = lv_bins(l);
    for (int i = threadIdx.x; i < nb; i += 64 * NW) sm.hist[i] = 0;
    __syncthreads();
    for (uint32_t e0 = 0; e0 < cnt; e0 += 64 * U) {
      uint32_t key[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = e0 + u * 64 + lane;
        key[u] = e < cnt ? key_of(e) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (e0 + u * 64 + lane < cnt && lv_in_range(key[u], l, prefix)) atomicAdd(&sm.hist[lv_digit(key[u], l)], 1u);
    }
    __syncthreads();
    find_bin_t<NW>(sm.hist, nb, need, sm);
    const uint32_t bin = sm.res[0], above = sm.res[1];
    __syncthreads();
    need -= above;
    prefix = (prefix << lv_bits(l)) | bin;
  }
  if (threadIdx.x == 0) {
    sm.res[0] = prefix;
    sm.res[1] = need;
  }
  __syncthreads();
}

template <typename KeyOf>
__device__ void radix_kth(KeyOf key_of, uint32_t cnt, int l0, uint32_t prefix, uint32_t need, SelSmem& sm) {
  radix_kth_t<SW>(key_of, cnt, l0, prefix, need, sm);
}

// Continue the radix search inside candidates (each wave owns [off, off+cnt)
// of cb) through levels lv+1..2.
__device__ void refine_candidates(const uint32_t* cb, uint32_t off, uint32_t cnt, int lv, uint32_t prefix,
                                  uint32_t need, SelSmem& sm) {
  radix_kth([&](uint32_t e) { return score_key(__uint_as_float(cb[off + e])); }, cnt, lv + 1, prefix, need, sm);
}

// The need-th largest key among candidates that are all >= lo (wave w owns cb[off, off + cnt)),
// with one histogram of NB0 bins over the candidates' own range [lo, max] (bins spread over the
// values actually present, so few atomics meet on one address), then the critical bin's
// elements ranked one by one. Result as for radix_kth: sm.res[0] = the need-th largest key T,
// sm.res[1] = how many keys == T to keep. Returns false, the result unset, when the critical
// bin holds more than REL_STASH elements (heavy ties): the caller takes the digit search.
constexpr uint32_t REL_STASH = 1024;
__device__ bool relative_kth(const uint32_t* cb, uint32_t off, uint32_t cnt, uint32_t lo, uint32_t need,
                             SelSmem& sm) {
  const int t = threadIdx.x, w = t >> 6, lane = lane_id();
  uint32_t mx = lo;
  for (uint32_t e = lane; e < cnt; e += 64) mx = max(mx, score_key(__uint_as_float(cb[off + e])));
  mx = wave_max_u32(mx);
  if (lane == 0) sm.gt[w] = mx;
  for (int i = t; i < NB0; i += ST) sm.hist[i] = 0;
  __syncthreads();
  uint32_t hi = lo;
#pragma unroll
  for (int i = 0; i < SW; ++i) hi = max(hi, sm.gt[i]);
  const uint32_t span = hi - lo;
  const int shift = span >= (uint32_t)NB0 ? (32 - __clz(span)) - 12 : 0;  // span >> shift < NB0
  for (uint32_t e = lane; e < cnt; e += 64)
    atomicAdd(&sm.hist[(score_key(__uint_as_float(cb[off + e])) - lo) >> shift], 1u);
  __syncthreads();
  find_bin_t<SW>(sm.hist, NB0, need, sm);
  const uint32_t bin = sm.res[0], above = sm.res[1], inbin = sm.hist[bin];
  __syncthreads();
  if (inbin > REL_STASH) return false;  // workgroup-uniform
  if (t == 0) sm.aux = 0u;
  __syncthreads();
  uint32_t* stash = sm.hist;  // the histogram is spent
  for (uint32_t e = lane; e < cnt; e += 64) {
    const uint32_t key = score_key(__uint_as_float(cb[off + e]));
    if (((key - lo) >> shift) == bin) stash[atomicAdd(&sm.aux, 1u)] = key;
  }
  __syncthreads();
  const uint32_t nd = need - above;  // 1 <= nd <= inbin
  for (uint32_t i = t; i < inbin; i += ST) {
    const uint32_t v = stash[i];
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < inbin; ++j) {
      const uint32_t x = stash[j];
      gt += x > v;
      ge += x >= v;
    }
    if (gt < nd && nd <= ge) {  // v is the nd-th largest of the bin (every such i writes the same)
      sm.res[0] = v;
      sm.res[1] = nd - gt;
    }
  }
  __syncthreads();
  return true;
}

// Emit, in position order, every element with key > T and the first need_eq
// elements with key == T. Wave w walks its own segment [0, cnt) through
// get(e) -> (bits, position); segments are in position order by wave.
template <typename Get, typename Sm>
__device__ void emit_segments(Get get, uint32_t cnt, uint32_t T, uint32_t need_eq, Sm& sm, int32_t* oidx,
                              float* osel, uint32_t kk) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  uint32_t ngt = 0, neq = 0;
  for (uint32_t e = lane; e < cnt; e += 64) {
    uint32_t bits;
    int32_t pos;
    get(e, bits, pos);
    const uint32_t key = score_key(__uint_as_float(bits));
    ngt += key > T;
    neq += key == T;
  }
  ngt = wave_sum(ngt);
  neq = wave_sum(neq);
  if (lane == 0) {
    sm.gt[w] = ngt;
    sm.eq[w] = neq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t eb = 0, ob = 0;
    for (int i = 0; i < SW; ++i) {
      sm.eqbase[i] = eb;
      sm.obase[i] = ob;
      const uint32_t take = need_eq > eb ? min(need_eq - eb, sm.eq[i]) : 0u;
      ob += sm.gt[i] + take;
      eb += sm.eq[i];
    }
  }
  __syncthreads();
  const uint32_t eqb = sm.eqbase[w];
  uint32_t run = sm.obase[w], eqrun = 0;
  for (uint32_t e0 = 0; e0 < cnt; e0 += 64) {
    const uint32_t e = e0 + lane;
    uint32_t bits = 0;
    int32_t pos = 0;
    const bool valid = e < cnt;
    if (valid) get(e, bits, pos);
    const uint32_t key = score_key(__uint_as_float(bits));
    const bool gt = valid && key > T;
    const bool eq = valid && key == T;
    const uint64_t be = ballot(eq);
    const uint32_t er = eqb + eqrun + count_below(be);
    const bool take = gt || (eq && er < need_eq);
    const uint64_t bs = ballot(take);
    const uint32_t slot = run + count_below(bs);
    if (take && slot < kk) {  // slot < kk always holds: exactly kk elements qualify
      oidx[slot] = pos;
      if (osel) osel[slot] = __uint_as_float(bits);
    }
    run += __popcll(bs);
    eqrun += __popcll(be);
  }
}

// ---------------------------------------------------------------------------
// Row mode: one workgroup per row. Dynamic LDS (smem_raw): SelSmem, then
// 4*capw candidate bits and 4*capw candidate positions.
// The k' = kk largest of the row s[0, n) (kk <= k, kk <= n) to oidx[0, k)
// (ascending, -1 after kk) and their scores to osel (if given). All 256
// threads of the workgroup call it; they leave it together.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void select_row_device(const float* __restrict__ s, int n, int64_t stride, int k, int kk,
                                                  int32_t* __restrict__ oidx, float* __restrict__ osel, int capw,
                                                  uint4* smem_raw) {
  SelSmem& sm = *reinterpret_cast<SelSmem*>(smem_raw);
  uint32_t* cb = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(smem_raw) + ((sizeof(SelSmem) + 15) & ~15));
  int32_t* cp = reinterpret_cast<int32_t*>(cb + 4 * capw);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  for (int j = kk + t; j < k; j += ST) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  if (kk <= 0) return;
  const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  const int seg = ((n + 4 * SW - 1) / (4 * SW)) * 4;
  const int r0 = min(n, w * seg), r1 = min(n, r0 + seg);
  if (kk == n) {
    for (int p = r0 + lane; p < r1; p += 64) {
      oidx[p] = p;
      if (osel) osel[p] = s[p];
    }
    return;
  }
  // Sampled threshold (long rows, k' <= n/8): the key T of the r-th largest of ns samples, r a
  // few standard deviations above the samples expected among the k' largest, so that one pass
  // collecting the keys >= T almost always yields between k' and the LDS capacity of them. Then
  // the k' largest are among them (the k'-th largest key is >= T) and the row is read once more
  // only when it is not so (the digit-by-digit search below).
  const int ns = min(SEL_SAMPLES, 4 * capw) & ~255;
  if (n >= SEL_SAMPLE_MIN_N && n <= SEL_SAMPLE_MAX_N && (int64_t)kk * 8 <= n && ns >= 1024 && aligned &&
      (n & 3) == 0 && (stride & 3) == 0) {
    // candidates as 4-byte keys and 16-bit offsets in the wave's segment (at most 65536 long)
    const uint32_t capf = (uint32_t)(capw * 8 / 6) & ~63u;
    uint16_t* cq = reinterpret_cast<uint16_t*>(cb + SW * capf);
    const int nch = ns / 64;  // chunks of 64 consecutive elements, spread over the row
    const int per_w = ns / SW;
    uint32_t* samp = cb;
    for (int c = w; c < nch; c += SW) {
      const int64_t at = (int64_t)c * n / nch;
      samp[c * 64 + lane] = score_key(s[at + lane]);
    }
    __syncthreads();
    const float E = (float)kk * (float)ns / (float)n;
    const uint32_t r = min((uint32_t)ns, (uint32_t)ceilf(E + 4.5f * sqrtf(E)) + 2u);
    // wave w owns the samples of chunks w, w + SW, ...
    radix_kth_t<SW>([&](uint32_t e) { return samp[((e >> 6) * SW + w) * 64 + (e & 63)]; }, (uint32_t)per_w, 0, 0u,
                    r, sm);
    const uint32_t T = sm.res[0];
    __syncthreads();  // every wave has T before the samples are overwritten
    const uint32_t c = collect_fast<SEL_U>(s, r0, r1, T, cb + w * capf, cq + w * capf, capf);
    if (lane == 0) sm.cnt[w] = c;
    __syncthreads();
    bool over = false;
    uint32_t base = 0, total = 0;
    for (int i = 0; i < SW; ++i) {
      over |= sm.cnt[i] > capf;
      base += (i < w) ? sm.cnt[i] : 0u;
      total += sm.cnt[i];
    }
    __syncthreads();
    if (total >= (uint32_t)kk && total <= SW * capf) {  // workgroup-uniform
      uint32_t off = w * capf;
      if (over) {  // uneven spread across waves: pack the waves' candidates back to back
        collect_fast<SEL_U>(s, r0, r1, T, cb + base, cq + base, 0xffffffffu);
        off = base;
        __syncthreads();
      }
      if (!relative_kth(cb, off, c, T, (uint32_t)kk, sm))
        radix_kth([&](uint32_t e) { return score_key(__uint_as_float(cb[off + e])); }, c, 0, 0u, (uint32_t)kk, sm);
      const uint32_t Tk = sm.res[0], need_eq = sm.res[1];
      __syncthreads();
      emit_segments([&](uint32_t e, uint32_t& bits, int32_t& pos) { bits = cb[off + e]; pos = r0 + (int)cq[off + e]; },
                    c, Tk, need_eq, sm, oidx, osel, (uint32_t)kk);
      return;
    }
  }
  int lv = 0;
  uint32_t prefix = 0, need = (uint32_t)kk, cnt_above = 0;
  while (true) {
    const int nb = lv_bins(lv);
    for (int i = t; i < nb; i += ST) sm.hist[i] = 0;
    __syncthreads();
    hist_pass(s, r0, r1, aligned, lv, prefix, sm.hist);
    __syncthreads();
    find_bin(sm.hist, nb, need, sm);
    const uint32_t bin = sm.res[0], above = sm.res[1];
    const uint32_t inbin = sm.hist[bin];
    __syncthreads();
    need -= above;
    cnt_above += above;
    prefix = (prefix << lv_bits(lv)) | bin;
    const uint32_t lo = prefix << lv_shift(lv);
    if (cnt_above + inbin <= (uint32_t)(SW * capw)) {
      uint32_t c = collect_pass(s, r0, r1, aligned, lo, cb + w * capw, cp + w * capw, (uint32_t)capw);
      if (lane == 0) sm.cnt[w] = c;
      __syncthreads();
      bool over = false;
      uint32_t base = 0;
      for (int i = 0; i < SW; ++i) {
        over |= sm.cnt[i] > (uint32_t)capw;
        base += (i < w) ? sm.cnt[i] : 0u;
      }
      uint32_t off = (uint32_t)(w * capw);
      if (over) {  // uneven spread across waves: pack the waves' candidates back to back
        collect_pass(s, r0, r1, aligned, lo, cb + base, cp + base, 0xffffffffu);
        off = base;
        __syncthreads();
      }
      refine_candidates(cb, off, c, lv, prefix, need, sm);
      const uint32_t T = sm.res[0], need_eq = sm.res[1];
      __syncthreads();
      emit_segments([&](uint32_t e, uint32_t& bits, int32_t& pos) { bits = cb[off + e]; pos = cp[off + e]; }, c, T,
                    need_eq, sm, oidx, osel, (uint32_t)kk);
      return;
    }
    if (lv == 2) {  // T fully known and still too many ties for LDS: stream the row
      emit_segments(
          [&](uint32_t e, uint32_t& bits, int32_t& pos) {
            pos = r0 + (int)e;
            bits = __float_as_uint(s[pos]);
          },
          (uint32_t)(r1 - r0), prefix, need, sm, oidx, osel, (uint32_t)kk);
      return;
    }
    ++lv;
  }
}

__global__ __launch_bounds__(256) void select_rows_kernel(const float* __restrict__ S, int n, int64_t stride, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ sel,
                                                          int capw, const uint32_t* __restrict__ row_flag,
                                                          const int32_t* __restrict__ krow) {
  if (row_flag && row_flag[blockIdx.x] == 0) return;  // only the rows flagged for a full select
  extern __shared__ uint4 smem_raw[];
  const int64_t row = blockIdx.x;
  const int kk = min(krow ? min(krow[row], k) : k, n);  // krow: a count per row, at most k (the row stride)
  select_row_device(S + row * stride, n, stride, k, kk, idx + row * k, sel ? sel + row * k : nullptr, capw, smem_raw);
}

// ---------------------------------------------------------------------------
// Short rows (n <= SH_NMAX) with k' <= 64: one wave per row, no workgroup
// barriers. Lane l holds positions j*64 + l. The k'-th largest of the lane
// maxima is a lower bound T0 of the row's k'-th largest key (the k' largest
// lane maxima are k' distinct elements, all >= T0), so every key of the
// answer, and every key tied with its last one, is >= T0. Those keys go to
// LDS in position order. With at most 64 of them (the usual case), each
// lane ranks its candidate against all others (larger key first, then lower
// position) and the k' best are emitted in position order; otherwise the
// exact k'-th key T comes from a most-significant-bit-first search whose
// counts are ballot popcounts, and the keys > T, then the first keys == T,
// are emitted.
// ---------------------------------------------------------------------------
constexpr int SH_PER = 32;             // keys per lane
constexpr int SH_NMAX = 64 * SH_PER;   // longest row
constexpr int SH_KMAX = 64;            // largest k

// Rank of this lane's value among the values of lanes 0..cnt-1 (larger first, lower lane first
// among equals). 64 independent lane reads: no serial chain of reductions.
__device__ __forceinline__ uint32_t wave_rank(uint32_t v, uint32_t cnt) {
  const uint32_t lane = (uint32_t)lane_id();
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
    r += ((uint32_t)j < cnt && (o > v || (o == v && (uint32_t)j < lane))) ? 1u : 0u;
  }
  return r;
}

// The k-th largest of the keys get(e), e < cnt, and in *need how many keys equal to it rank among
// the k largest (k - the count of larger keys).
template <typename Get>
__device__ uint32_t wave_kth(Get get, uint32_t cnt, uint32_t k, uint32_t* need) {
  uint32_t prefix = 0, rem = k;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t hi = ~0u << bit;  // the bits decided so far and this one
    const uint32_t want = prefix | (1u << bit);
    uint32_t c = 0;
    for (uint32_t e0 = 0; e0 < cnt; e0 += 64) {
      const uint32_t e = e0 + (uint32_t)lane_id();
      c += (uint32_t)__popcll(ballot(e < cnt && (get(e) & hi) == want));
    }
    if (c >= rem) prefix = want;
    else rem -= c;
  }
  *need = rem;
  return prefix;
}

__global__ __launch_bounds__(256) void select_short_kernel(const float* __restrict__ S, int64_t n_rows, int n,
                                                           int64_t stride, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ sel) {
  __shared__ uint32_t cbits[4][SH_NMAX];
  __shared__ uint16_t cpos[4][SH_NMAX];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= n_rows) return;  // wave-uniform; nothing below waits for other waves
  const float* s = S + row * stride;
  int32_t* oidx = idx + row * k;
  float* osel = sel ? sel + row * k : nullptr;
  const int kk = min(k, n);
  for (int j = kk + lane; j < k; j += 64) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  if (kk <= 0) return;
  uint32_t bits[SH_PER], key[SH_PER];
#pragma unroll
  for (int j = 0; j < SH_PER; ++j) {
    const int p = j * 64 + lane;
    bits[j] = p < n ? __float_as_uint(s[p]) : 0u;
  }
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < SH_PER; ++j) {
    key[j] = score_key(__uint_as_float(bits[j]));
    if (j * 64 + lane < n) lm = max(lm, key[j]);
  }
  // lanes holding a key: min(64, n) >= kk; T0 = the lane maximum ranked kk - 1
  const uint32_t nl = (uint32_t)min(64, n);
  const uint64_t at = ballot((uint32_t)lane < nl && wave_rank(lm, nl) == (uint32_t)kk - 1);
  const uint32_t T0 = (uint32_t)__builtin_amdgcn_readlane((int)lm, (int)__builtin_ctzll(at));
  uint32_t C = 0;
#pragma unroll
  for (int j = 0; j < SH_PER; ++j) {
    const int p = j * 64 + lane;
    const bool take = p < n && key[j] >= T0;
    const uint64_t b = ballot(take);
    if (take) {
      const uint32_t slot = C + (uint32_t)count_below(b);
      cbits[w][slot] = bits[j];
      cpos[w][slot] = (uint16_t)p;
    }
    C += (uint32_t)__popcll(b);
  }
  lds_wave_sync();
  if (C <= 64) {  // candidate e on lane e, already in position order
    const bool ok = lane < (int)C;
    const uint32_t b = ok ? cbits[w][lane] : 0u;
    const bool take = ok && wave_rank(score_key(__uint_as_float(b)), C) < (uint32_t)kk;
    const uint64_t bs = ballot(take);
    if (take) {
      const uint32_t slot = (uint32_t)count_below(bs);
      oidx[slot] = cpos[w][lane];
      if (osel) osel[slot] = __uint_as_float(b);
    }
    return;
  }
  uint32_t need;
  const uint32_t T =
      wave_kth([&](uint32_t e) { return score_key(__uint_as_float(cbits[w][e])); }, C, (uint32_t)kk, &need);
  uint32_t run = 0, eqrun = 0;
  for (uint32_t e0 = 0; e0 < C; e0 += 64) {
    const uint32_t e = e0 + (uint32_t)lane;
    const bool ok = e < C;
    const uint32_t b = ok ? cbits[w][e] : 0u;
    const uint32_t kv = score_key(__uint_as_float(b));
    const bool gt = ok && kv > T, eq = ok && kv == T;
    const uint64_t be = ballot(eq);
    const bool take = gt || (eq && eqrun + (uint32_t)count_below(be) < need);
    const uint64_t bs = ballot(take);
    if (take) {  // exactly kk keys qualify
      const uint32_t slot = run + (uint32_t)count_below(bs);
      oidx[slot] = cpos[w][e];
      if (osel) osel[slot] = __uint_as_float(b);
    }
    run += (uint32_t)__popcll(bs);
    eqrun += (uint32_t)__popcll(be);
  }
}

// ---------------------------------------------------------------------------
// Split mode (few long rows)
// ---------------------------------------------------------------------------
__global__ void select_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ __launch_bounds__(256) void select_chunk_hist_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                                int k, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[NB0];
  const int64_t row = blockIdx.y;
  if (min(k, n) == n) return;
  const float* s = S + row * stride;
  const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  const int w = threadIdx.x >> 6;
  const int c0 = blockIdx.x * CHUNK;
  const int r0 = min(n, c0 + w * SUBCH), r1 = min(n, r0 + SUBCH);
  for (int i = threadIdx.x; i < NB0; i += ST) hist[i] = 0;
  __syncthreads();
  hist_pass(s, r0, r1, aligned, 0, 0, hist);
  __syncthreads();
  uint32_t* gh = ghist + row * NB0;
  for (int i = threadIdx.x; i < NB0; i += ST)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// Level-1 digits of the keys inside the level-0 bin that holds the k'-th key.
__global__ __launch_bounds__(256) void select_chunk_hist1_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                                 int k, const uint32_t* __restrict__ ghist,
                                                                 uint32_t* __restrict__ ghist1) {
  __shared__ SelSmem sm;
  const int64_t row = blockIdx.y;
  const int kk = min(k, n);
  if (kk == n) return;
  const float* s = S + row * stride;
  const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  const uint32_t* gh = ghist + row * NB0;
  for (int i = threadIdx.x; i < NB0; i += ST) sm.hist[i] = gh[i];
  __syncthreads();
  find_bin(sm.hist, NB0, (uint32_t)kk, sm);
  const uint32_t bin0 = sm.res[0];
  __syncthreads();
  for (int i = threadIdx.x; i < NB1; i += ST) sm.hist[i] = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6;
  const int c0 = blockIdx.x * CHUNK;
  const int r0 = min(n, c0 + w * SUBCH), r1 = min(n, r0 + SUBCH);
  hist_pass(s, r0, r1, aligned, 1, bin0, sm.hist);
  __syncthreads();
  uint32_t* g1 = ghist1 + row * NB1;
  for (int i = threadIdx.x; i < NB1; i += ST)
    if (sm.hist[i]) atomicAdd(&g1[i], sm.hist[i]);
}

// The level-0 and level-1 bins that hold the k'-th key of a row, from the global histograms:
// (bin0, bin1) and the counts of keys above each.
__device__ void split_bins(const uint32_t* gh0, const uint32_t* gh1, uint32_t kk, SelSmem& sm, uint32_t* bin0,
                           uint32_t* above0, uint32_t* bin1, uint32_t* above1) {
  for (int i = threadIdx.x; i < NB0; i += ST) sm.hist[i] = gh0[i];
  __syncthreads();
  find_bin(sm.hist, NB0, kk, sm);
  *bin0 = sm.res[0];
  *above0 = sm.res[1];
  __syncthreads();
  for (int i = threadIdx.x; i < NB1; i += ST) sm.hist[i] = gh1[i];
  __syncthreads();
  find_bin(sm.hist, NB1, kk - *above0, sm);
  *bin1 = sm.res[0];
  *above1 = sm.res[1];
  __syncthreads();
}

__global__ __launch_bounds__(256) void select_chunk_collect_kernel(const float* __restrict__ S, int n,
                                                                   int64_t stride, int k,
                                                                   const uint32_t* __restrict__ ghist,
                                                                   const uint32_t* __restrict__ ghist1,
                                                                   uint32_t* __restrict__ cbits,
                                                                   int32_t* __restrict__ cpos,
                                                                   uint32_t* __restrict__ ccount, int nch) {
  __shared__ SelSmem sm;
  const int64_t row = blockIdx.y;
  const int kk = min(k, n);
  if (kk == n) return;
  const float* s = S + row * stride;
  const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  uint32_t bin0, above0, bin1, above1;
  split_bins(ghist + row * NB0, ghist1 + row * NB1, (uint32_t)kk, sm, &bin0, &above0, &bin1, &above1);
  const uint32_t lo = (bin0 << 20) | (bin1 << 10);  // keys at or above the level-1 bin of the k'-th key
  const int w = threadIdx.x >> 6;
  const int c0 = blockIdx.x * CHUNK;
  const int r0 = min(n, c0 + w * SUBCH), r1 = min(n, r0 + SUBCH);
  const int64_t base = row * (int64_t)n + r0;
  const uint32_t c = collect_pass(s, r0, r1, aligned, lo, cbits + base, cpos + base, (uint32_t)SUBCH);
  if (lane_id() == 0) ccount[(row * nch + blockIdx.x) * SW + w] = c;
}

// Dynamic LDS: nseg segment offsets, then room for lcap candidates (bits, positions).
constexpr int FIN_LDS_CAP = 4096;
constexpr size_t FIN_DYN_MAX = 65536 - sizeof(SelSmem) - 256;  // dynamic LDS beside the static part
__global__ __launch_bounds__(256) void select_finish_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                            int k, const uint32_t* __restrict__ ghist,
                                                            const uint32_t* __restrict__ ghist1,
                                                            const uint32_t* __restrict__ cbits,
                                                            const int32_t* __restrict__ cpos,
                                                            const uint32_t* __restrict__ ccount,
                                                            uint32_t* __restrict__ catb, int32_t* __restrict__ catp,
                                                            int nch, int32_t* __restrict__ idx,
                                                            float* __restrict__ sel, int lcap) {
  __shared__ SelSmem sm;
  extern __shared__ uint32_t segoff[];
  const int64_t row = blockIdx.x;
  const float* s = S + row * stride;
  int32_t* oidx = idx + row * k;
  float* osel = sel ? sel + row * k : nullptr;
  const int kk = min(k, n);
  const int t = threadIdx.x, w = t >> 6;
  for (int j = kk + t; j < k; j += ST) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  if (kk <= 0) return;
  if (kk == n) {
    for (int p = t; p < n; p += ST) {
      oidx[p] = p;
      if (osel) osel[p] = s[p];
    }
    return;
  }
  uint32_t bin0, above0, bin1, above1;
  split_bins(ghist + row * NB0, ghist1 + row * NB1, (uint32_t)kk, sm, &bin0, &above0, &bin1, &above1);
  const uint32_t prefix = (bin0 << 10) | bin1, above = above0 + above1;
  // offsets of the (chunk, wave) segments, in position order
  const int nseg = nch * SW;
  const uint32_t* cc = ccount + row * (int64_t)nseg;
  const int per = (nseg + ST - 1) / ST;
  uint32_t loc = 0;
  for (int i = 0; i < per; ++i) {
    const int sg = t * per + i;
    loc += sg < nseg ? cc[sg] : 0u;
  }
  uint32_t total;
  const uint32_t incl = block_incl_scan(loc, sm, &total);
  uint32_t run = incl - loc;
  for (int i = 0; i < per; ++i) {
    const int sg = t * per + i;
    if (sg < nseg) {
      segoff[sg] = run;
      run += cc[sg];
    }
  }
  __syncthreads();
  // concatenate the segments in position order: output e comes from the last segment whose
  // offset is <= e (binary search over the offsets; independent loads across threads), into
  // LDS after the offsets when they fit (the refinement and the emission then read LDS), else
  // into the row's global scratch
  auto tail = [&](uint32_t* rb, int32_t* rp) {
    for (uint32_t e = t; e < total; e += ST) {
      int lo = 0, hi = nseg - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segoff[mid] <= e) lo = mid;
        else hi = mid - 1;
      }
      const int64_t src = row * (int64_t)n + (int64_t)(lo / SW) * CHUNK + (lo % SW) * SUBCH + (e - segoff[lo]);
      rb[e] = cbits[src];
      rp[e] = cpos[src];
    }
    __syncthreads();
    const uint32_t q = (total + SW - 1) / SW;
    const uint32_t off = min(total, (uint32_t)w * q);
    const uint32_t cnt = min(total, off + q) - off;
    refine_candidates(rb, off, cnt, 1, prefix, (uint32_t)kk - above, sm);
    const uint32_t T = sm.res[0], need_eq = sm.res[1];
    __syncthreads();
    emit_segments([&](uint32_t e, uint32_t& bits, int32_t& pos) { bits = rb[off + e]; pos = rp[off + e]; }, cnt,
                  T, need_eq, sm, oidx, osel, (uint32_t)kk);
  };
  if (total <= (uint32_t)lcap)  // workgroup-uniform
    tail(segoff + nseg, reinterpret_cast<int32_t*>(segoff + nseg + lcap));
  else
    tail(catb + row * (int64_t)n, catp + row * (int64_t)n);
}

// ---------------------------------------------------------------------------
// Candidate prefilter for the fused exact step. A sampled scoring pass gives
// each row a key threshold T (the r-th largest sample key); the scan keeps
// only scores with key >= T. If at least k' of them were kept, every one of
// the k' largest keys is among them (the k'-th largest key is then >= T), so
// the exact answer comes from the candidates alone; otherwise the row is
// flagged and rescored in full.
// ---------------------------------------------------------------------------
#ifndef TKA_PF_NW
#define TKA_PF_NW 16
#endif
#ifndef TKA_PF_MINW
#define TKA_PF_MINW 8
#endif
constexpr int PF_NW = TKA_PF_NW;  // waves of the finish kernel (one row per workgroup)
constexpr int PF_T = 64 * PF_NW;
constexpr int PF_RC = 12288 / PF_T;  // candidates held per thread: capacity <= 12288

constexpr int PF_STASH = 2048;  // elements of the critical bin ranked one by one
#ifndef TKA_PF_REPAIR_BYTES
#define TKA_PF_REPAIR_BYTES (64ll << 20)
#endif
constexpr long long PF_REPAIR_BYTES = TKA_PF_REPAIR_BYTES;  // score slots of the repair kernel

struct PfSmem {
  uint32_t skey[PF_STASH];
  uint32_t sidx[PF_STASH];
  int32_t spos[PF_STASH];
  uint32_t scnt;
  uint32_t red[PF_NW];
};
// the finish emits up to PF_KMAX kept pairs through the spent histogram and stash keys
constexpr int PF_KMAX = 4096;
static_assert(NB0 >= PF_KMAX && 2 * PF_STASH >= PF_KMAX &&
                  offsetof(PfSmem, sidx) == offsetof(PfSmem, skey) + sizeof(uint32_t) * PF_STASH,
              "finish emission staging");

// Threshold of a row: the key of its r-th largest sample. One wave per row,
// the row's samples held in registers (RS per lane, lane-strided). Radix
// levels of 1024 bins over the current key range [lo, lo + span]: the bin
// holding the r-th key (counting from the top) becomes the next range, until
// it is one key wide or holds at most 64 samples, which are then ranked one
// by one. The result is exact: every level narrows the range by 2^10. The
// wave also clears the row's counters and flags. No workgroup barriers.
template <int RS>
__global__ __launch_bounds__(256) void prefilter_threshold_kernel(const float* __restrict__ samp, int nsamp, int r,
                                                                  int64_t n_rows, float* __restrict__ T,
                                                                  uint32_t* __restrict__ cnt,
                                                                  uint32_t* __restrict__ row_flag,
                                                                  uint32_t* __restrict__ group_flag, int G, int Hq,
                                                                  int M) {
  __shared__ uint32_t hist_all[4][1024];
  __shared__ uint32_t list_all[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= n_rows) return;
  uint32_t* hist = hist_all[w];
  uint32_t* lst = list_all[w];
  if (lane == 0) {
    cnt[row] = 0;
    row_flag[row] = 0;
    // rows (b, t, h), several queries t per sequence: the group flag of (b, h / G) is cleared once
    if ((row / Hq) % M == 0 && (row % Hq) % G == 0) group_flag[(row / ((int64_t)M * Hq)) * (Hq / G) + (row % Hq) / G] = 0;
  }
  if (r > nsamp) {
    if (lane == 0) T[row] = key_value(0u);  // too few samples: keep everything
    return;
  }
  const float* s = samp + row * nsamp;
  uint32_t key[RS];
  uint32_t mn = 0xffffffffu, mx = 0u;
  float raw[RS];
#pragma unroll
  for (int j = 0; j < RS; ++j) raw[j] = s[min(lane + 64 * j, nsamp - 1)];  // all loads in flight together
#pragma unroll
  for (int j = 0; j < RS; ++j) {
    const bool ok = lane + 64 * j < nsamp;
    key[j] = ok ? score_key(raw[j]) : 0u;
    mn = ok ? min(mn, key[j]) : mn;
    mx = ok ? max(mx, key[j]) : mx;
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  uint32_t lo = mn, span = mx - mn, need = (uint32_t)r, result = mn;
  for (;;) {
    const int shift = span >= 1024u ? (32 - __clz(span)) - 10 : 0;  // span >> shift < 1024
#pragma unroll
    for (int i = 0; i < 16; ++i) hist[lane + 64 * i] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < RS; ++j)
      if (lane + 64 * j < nsamp && key[j] - lo <= span) atomicAdd(&hist[(key[j] - lo) >> shift], 1u);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    // lane l owns bins [16 l, 16 l + 16); counts above a lane's bins from a prefix over lanes
    uint32_t c[16], sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      c[i] = hist[16 * lane + i];
      sum += c[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t above = tot - incl;
    const uint64_t hit = ballot(above < need && need <= above + sum);
    if (hit == 0) {  // not reached: 1 <= need <= tot at every level
      result = lo;
      break;
    }
    const int h = (int)__builtin_ctzll(hit);
    uint32_t bin = 0, abv = 0;
    if (lane == h) {
      uint32_t acc = above;
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        if (acc + c[i] >= need) {
          bin = 16 * lane + i;
          abv = acc;
          break;
        }
        acc += c[i];
      }
    }
    bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, h);
    abv = (uint32_t)__builtin_amdgcn_readlane((int)abv, h);
    need -= abv;  // rank of the answer inside the bin, from its top
    const uint32_t blo = lo + (bin << shift);
    if (shift == 0) {  // one key wide
      result = blo;
      break;
    }
    const uint32_t inbin = hist[bin];
    if (inbin <= 64u) {  // rank the bin's samples one by one
      uint32_t base = 0;
#pragma unroll
      for (int j = 0; j < RS; ++j) {
        const bool in = lane + 64 * j < nsamp && key[j] - lo <= span && ((key[j] - lo) >> shift) == bin;
        const uint64_t m = ballot(in);
        if (in) lst[base + count_below(m)] = key[j];
        base += (uint32_t)__builtin_popcountll(m);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      const uint32_t v = lane < (int)inbin ? lst[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (uint32_t u = 0; u < inbin; ++u) {
        const uint32_t x = lst[u];
        gt += x > v;
        ge += x >= v;
      }
      const uint64_t ok = ballot(lane < (int)inbin && gt < need && need <= ge);
      result = ok ? (uint32_t)__builtin_amdgcn_readlane((int)v, (int)__builtin_ctzll(ok)) : blo;
      break;
    }
    lo = blo;
    span = (1u << shift) - 1u;
    __builtin_amdgcn_wave_barrier();  // this level's bin reads precede the next level's clearing
  }
  if (lane == 0) T[row] = key_value(result);
}

// An empty asm that takes v in a VGPR and may change it: the value is materialised here, and
// nothing computed from it before is reused after (so its register is the only one kept live).
template <typename T>
__device__ __forceinline__ void pin_vgpr(T& v) {
  asm volatile("" : "+v"(v));
}

// Exact top-k of a row from its (unordered) candidates, whose keys are all
// >= T[row]. One relative-digit histogram finds the bin holding the k'-th
// key; its few elements are ranked one by one (key, then lower position
// first). Kept positions are marked in an LDS bitmap over the row and
// popcount prefix sums give each its output slot in ascending position
// order. Dynamic LDS: 2 * ceil(n/32) words (kept bitmap, prefix counts).
// Thread t holds candidates t + PF_T j, j < PF_RC, with their keys computed
// once. The valid elements of a wave are a prefix of j (only the last can be
// valid on part of the wave), so each per-element pass stops at the wave's
// count and takes the partial element without a branch: a lane's invalid
// element adds to a dummy bin of its own and ORs zero into the bitmap. (With
// 16 waves per row and two rows per CU, the exec-mask branches of a plain
// per-element loop made these passes scalar-issue bound.)
__global__ __launch_bounds__(PF_T, TKA_PF_MINW) void prefilter_finish_kernel(const uint2* __restrict__ cpair,
                                                                const uint32_t* __restrict__ cnt,
                                                                const float* __restrict__ Tv, int capg, int n,
                                                                int k, int G, int Hq, int M,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ sel,
                                                                uint32_t* __restrict__ row_flag,
                                                                uint32_t* __restrict__ group_flag) {
  __shared__ SelSmem sm;
  __shared__ PfSmem ps;
  extern __shared__ uint4 dyn4[];  // 16-byte aligned
  uint32_t* dyn = reinterpret_cast<uint32_t*>(dyn4);
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63;
  const int kk = min(k, n);
  int32_t* oidx = idx + row * k;
  float* osel = sel ? sel + row * k : nullptr;
  for (int j = kk + t; j < k; j += PF_T) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  const uint32_t nc = cnt[row];
  // threshold too high, or too many candidates (or more kept than the emission stages: the
  // prefilter's plan never asks for that)
  bool repair = nc < (uint32_t)kk || nc > (uint32_t)capg || kk > PF_KMAX;
  if (!repair) {
    const u32x2_t* cw = reinterpret_cast<const u32x2_t*>(cpair + row * capg);
    const uint32_t T0 = score_key(Tv[row]);
    // the thread's candidates, every load of the batch in flight together (indices past the
    // count re-read the last candidate and are marked invalid: position -1, key T0)
    u32x2_t x[PF_RC];
#pragma unroll
    for (int j = 0; j < PF_RC; ++j) x[j] = cw[min((uint32_t)(t + PF_T * j), nc - 1u)];  // (score bits, position)
    // the scores are kept as their keys, whose inverse gives back every score's bits except a
    // NaN's payload and the sign of -0 (keys 0 and 0x80000000: those are re-read at emission)
    uint32_t key[PF_RC];
    int32_t pos[PF_RC];
#pragma unroll
    for (int j = 0; j < PF_RC; ++j) {
      const bool ok = (uint32_t)(t + PF_T * j) < nc;
      const uint32_t kv = score_key(__uint_as_float(x[j][0]));  // computed for every lane: a select, no branch
      pos[j] = ok ? (int32_t)x[j][1] : -1;
      key[j] = ok ? kv : T0;
      pin_vgpr(pos[j]);
      pin_vgpr(key[j]);
    }
    const int words = (n + 31) >> 5;
    uint32_t* bm = dyn;
    uint32_t* pre = dyn + words;
    // one barrier for the cleared bitmap and histogram and the waves' maxima (every key is >= T0,
    // so the candidates' range is [T0, max])
    // 16-byte stores (the dynamic area holds whole quads: up to three words of pre are cleared too)
    for (int i = t; i < (words + 3) / 4; i += PF_T) dyn4[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = t; i < NB0 / 4; i += PF_T) reinterpret_cast<uint4*>(sm.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) ps.scnt = 0;
    uint32_t mx = T0;
#pragma unroll
    for (int j = 0; j < PF_RC; ++j) mx = max(mx, key[j]);
    mx = wave_max_u32(mx);
    if (lane == 0) ps.red[t >> 6] = mx;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PF_NW; ++i) mx = max(mx, ps.red[i]);
    const uint32_t span = mx - T0;
    const int shift = span >= 4096u ? (32 - __clz(span)) - 12 : 0;  // span >> shift < 4096
#pragma unroll
    for (int j = 0; j < PF_RC; ++j)
      if (pos[j] >= 0) atomicAdd(&sm.hist[(key[j] - T0) >> shift], 1u);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PF_RC; ++j) pin_vgpr(key[j]);  // digits recomputed below, not held
    find_bin_t<PF_NW>(sm.hist, NB0, (uint32_t)kk, sm);
    // (bin and rank in SGPRs: no LDS wait inside the passes below)
    const uint32_t bin = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.res[0]);
    const uint32_t need = (uint32_t)kk - (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.res[1]);
    // keys above the critical bin are kept; the bin's elements go to the stash
#pragma unroll
    for (int j = 0; j < PF_RC; ++j) {
      const int32_t p = pos[j];
      const uint32_t d = (key[j] - T0) >> shift;
      if (p >= 0 && d > bin) atomicOr(&bm[p >> 5], 1u << (p & 31));
      const bool eq = p >= 0 && d == bin;
      const uint64_t me = ballot(eq);
      if (__builtin_expect(me != 0, 0)) {  // wave-uniform: one reservation for the wave's stash entries
        const int first = (int)__builtin_ctzll(me);
        uint32_t base = 0;
        if (lane == first) base = atomicAdd(&ps.scnt, (uint32_t)__builtin_popcountll(me));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
        const uint32_t slot = base + (uint32_t)count_below(me);
        if (eq && slot < PF_STASH) {
          ps.skey[slot] = key[j];
          ps.spos[slot] = p;
        }
      }
    }
    __syncthreads();
    const uint32_t m = ps.scnt;
    repair = m > PF_STASH;  // heavy ties in one bin: leave the row to the full select
    if (!repair) {
      for (uint32_t i = t; i < m; i += PF_T) {
        const uint32_t v = ps.skey[i];
        const int32_t pv = ps.spos[i];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < m; ++u) rank += ps.skey[u] > v || (ps.skey[u] == v && ps.spos[u] < pv);
        if (rank < need) atomicOr(&bm[pv >> 5], 1u << (pv & 31));
      }
      __syncthreads();
      const int per = (words + PF_T - 1) / PF_T;
      uint32_t loc = 0;
      for (int i = 0; i < per; ++i) {
        const int wd = t * per + i;
        loc += wd < words ? __popc(bm[min(wd, words - 1)]) : 0u;
      }
      uint32_t total;
      uint32_t run = block_incl_scan_t<PF_NW, SelSmem, false>(loc, sm, &total) - loc;  // closed by the barrier below
      for (int i = 0; i < per; ++i) {
        const int wd = t * per + i;
        if (wd < words) {
          pre[wd] = run;
          run += __popc(bm[wd]);
        }
      }
      __syncthreads();
      // the kept pairs to their slots in LDS (the histogram and the stash are spent: k' <= 4096
      // entries each), then out with 16-byte stores in slot order; a candidate is kept exactly
      // when its bit is set (each position is a candidate once)
      uint32_t* lidx = sm.hist;
      uint32_t* lsel = ps.skey;  // skey and sidx: 2 * PF_STASH contiguous entries
#pragma unroll
      for (int j = 0; j < PF_RC; ++j) {
        const int32_t p = pos[j];
        const uint32_t kj = key[j];
        if (p < 0 || ((kj - T0) >> shift) < bin) continue;
        const uint32_t word = bm[p >> 5], bit = (uint32_t)p & 31u;
        if (!((word >> bit) & 1u)) continue;
        const uint32_t slot = pre[p >> 5] + __popc(word & ((1u << bit) - 1u));
        if (slot < (uint32_t)kk) {
          uint32_t sb = (kj & 0x80000000u) ? (kj & 0x7fffffffu) : ~kj;  // the key's inverse
          if ((kj & 0x7fffffffu) == 0u) sb = cw[t + PF_T * j][0];          // a NaN or a zero: its own bits
          lidx[slot] = (uint32_t)p;
          lsel[slot] = sb;
        }
      }
      __syncthreads();
      const bool vec = ((reinterpret_cast<uintptr_t>(oidx) | reinterpret_cast<uintptr_t>(osel)) & 15) == 0;
      for (int i = 4 * t; i < kk; i += 4 * PF_T) {
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
  }
  if (repair && t == 0) {
    row_flag[row] = 1u;
    atomicOr(&group_flag[(row / ((int64_t)M * Hq)) * (Hq / G) + (row % Hq) / G], 1u);  // group (b, h / G)
  }
}

// ---------------------------------------------------------------------------
// Repair of the rows the prefilter flagged (the answer is not certainly among
// a row's candidates): the row's exact scores, then the row select over them.
// Persistent, nslot workgroups, each with its own slot of min(16, R) score
// rows (R = M*G rows per group, below): the
// flagged (b, KV head) groups are taken in order, the i-th by workgroup
// i % nslot, with no waits between workgroups. A group's R = M*G (query,
// head) rows are scored in blocks of 16 (skipping blocks with no flagged
// row) with the scorers' arithmetic: v_mfma_f32_16x16x32_bf16 over the same
// operand layout and 32-dim step order (A = 16 key rows staged through LDS,
// B = the block's query rows, one per column), times the scale, positions a
// query cannot see set to NaN, so the slot holds bitwise what
// topk_attn_score writes for those rows; each flagged row of the block is
// then selected from its slot row with k' = min(k, its visible keys).
// On a step with no flagged group every workgroup reads the group flags and
// leaves. Dynamic LDS: max(4 waves x 32 staged rows, the row select's).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefilter_repair_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ K, int Hq, int Hkv, int G,
                                                               int M, int L, int64_t sb, int64_t sh, int64_t sl,
                                                               float scale, int k, int n_groups,
                                                               const uint32_t* __restrict__ group_flag,
                                                               const uint32_t* __restrict__ row_flag,
                                                               float* __restrict__ slots, int32_t* __restrict__ idx,
                                                               float* __restrict__ sel, int capw) {
  constexpr int KS = D / 32;
  constexpr int P = 32;  // positions per wave round (two 16-position MFMA tiles)
  constexpr int RB = D * 2, PADB = RB + 16, CPR = RB / 16, RPI = 1024 / RB, NI = P / RPI;
  extern __shared__ uint4 smem_raw[];
  __shared__ int32_t mine[256];  // flagged groups of this workgroup, in order
  __shared__ uint32_t wcnt[SW];
  __shared__ int32_t nmine_s;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int nslot = (int)gridDim.x, me = (int)blockIdx.x;
  const int R = M * G;
  float* slot = slots + (size_t)me * min(16, R) * (size_t)L;  // min(16, R) score rows per slot

  // this workgroup's flagged groups: ranks among the flagged groups by ballots and a scan over waves
  if (t == 0) nmine_s = 0;
  uint32_t rank0 = 0;  // flagged groups before the current window of 256
  for (int g0 = 0; g0 < n_groups; g0 += 256) {
    const int gi = g0 + t;
    const bool f = gi < n_groups && group_flag[gi] != 0u;
    const uint64_t bl = ballot(f);
    if (lane == 0) wcnt[wave] = (uint32_t)__popcll(bl);
    __syncthreads();
    uint32_t before = rank0 + (uint32_t)count_below(bl), tot = 0;
    for (int i = 0; i < SW; ++i) {
      before += i < wave ? wcnt[i] : 0u;
      tot += wcnt[i];
    }
    if (f && (int)(before % (uint32_t)nslot) == me) {
      const int at = (int)(before / (uint32_t)nslot);
      if (at < 256) mine[at] = gi;
      atomicMax(&nmine_s, at + 1);
    }
    rank0 += tot;
    __syncthreads();
  }
  const int nmine = min(nmine_s, 256);  // groups beyond 256 per workgroup: the plan keeps n_groups <= 256 * nslot
  uint8_t* stage = reinterpret_cast<uint8_t*>(smem_raw) + (size_t)wave * P * PADB;

  for (int mi = 0; mi < nmine; ++mi) {
    const int grp = mine[mi];
    const int b = grp / Hkv, g = grp % Hkv;
    const uint16_t* Kb = K + (int64_t)b * sb + (int64_t)g * sh;
    for (int cb = 0; cb * 16 < R; ++cb) {
      // flagged rows of the block (every wave computes the same mask)
      const int rl = cb * 16 + (lane & 15);
      const bool rin = lane < 16 && rl < R;
      const int64_t rrow = ((int64_t)b * M + (rin ? rl / G : 0)) * Hq + g * G + (rin ? rl % G : 0);
      const uint64_t fm = ballot(rin && row_flag[rrow] != 0u);
      if (fm == 0) continue;  // workgroup-uniform
      // score the block's rows over every position into the slot
      const int rr = cb * 16 + n;
      const bool ok = rr < R;
      const int tq = ok ? rr / G : 0, hh = ok ? rr % G : 0;
      const int64_t qr = ((int64_t)b * M + tq) * Hq + g * G + hh;
      const int last = L - M + tq;  // the last position the row's query sees
      bf16x8_t bq[KS];
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = ld16(q + qr * D + 32 * s2 + 8 * kg);
        bq[s2] = __builtin_bit_cast(bf16x8_t, v);
      }
      float* srow = slot + (size_t)n * L;
      auto load = [&](uint4 (&a)[NI], int at) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int pos = min(at + j * RPI + lane / CPR, L - 1);
          a[j] = ld16(Kb + (int64_t)pos * sl + (lane % CPR) * 8);
        }
      };
      int base = wave * P;
      uint4 cur[NI];
      if (base < L) load(cur, base);
      for (; base < L; base += 4 * P) {
        uint4 nxt[NI];
        const bool more = base + 4 * P < L;
        if (more) load(nxt, base + 4 * P);
#pragma unroll
        for (int j = 0; j < NI; ++j)
          *reinterpret_cast<uint4*>(stage + (j * RPI + lane / CPR) * PADB + (lane % CPR) * 16) = cur[j];
        lds_wave_sync();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) {
            const uint4 a = *reinterpret_cast<const uint4*>(stage + (16 * tt + n) * PADB + (kg + 4 * s2) * 16);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bq[s2], acc, 0, 0, 0);
          }
          const int pos = base + 16 * tt + 4 * kg;
          if (ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (pos + i < L) srow[pos + i] = pos + i <= last ? acc[i] * scale : __int_as_float(0x7fc00000);
          }
        }
        __builtin_amdgcn_wave_barrier();  // reads of this round precede the next writes
        if (more) {
#pragma unroll
          for (int j = 0; j < NI; ++j) cur[j] = nxt[j];
        }
      }
      __syncthreads();  // the slot's scores are written (and the staging area is free)
      for (uint64_t m = fm; m != 0; m &= m - 1) {
        const int j = (int)__builtin_ctzll(m);
        const int r2 = cb * 16 + j, t2 = r2 / G;
        const int64_t row = ((int64_t)b * M + t2) * Hq + g * G + r2 % G;
        const int kk = min(k, L - M + t2 + 1);
        select_row_device(slot + (size_t)j * L, L, L, k, kk, idx + row * k, sel ? sel + row * k : nullptr, capw,
                          smem_raw);
        __syncthreads();  // the select's LDS and slot reads are done
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The indexer variant's fused select (few long rows: one kept set per
// sequence, "Sparse Attention in LLM Inference", "The Role of the Indexer").
// The scoring pass keeps, for every chunk of IC positions, the chunk's IC_KEEP
// first positions in the select order as candidates, in position order, at
// fixed slots (no counters). One workgroup per sequence then selects the k'
// first candidates. That is the exact answer unless some chunk could hold a
// kept position beyond its candidates: every candidate of a chunk kept means
// its worst candidate is kept, so a chunk whose smallest candidate key is at
// least the k'-th key T (ties included, conservatively) sends the row to the
// full row select over the score array. The k' first positions overall that
// are candidates are the k' first candidates; if one position were missing, it
// would lie in a chunk whose candidates are all ahead of it, and all kept.
// ---------------------------------------------------------------------------
constexpr int IC = 2048;           // positions per chunk (one scoring workgroup)
constexpr int IC_KEEP = 16;        // candidates per chunk
constexpr int IC_CAND_MAX = 16384;  // candidates per sequence the finish holds in registers
template <int DI, int NT>
__global__ __launch_bounds__(256) void indexer_cand_kernel(const uint8_t* __restrict__ qI,
                                                           const uint8_t* __restrict__ kI,
                                                           const float* __restrict__ w, float* __restrict__ S,
                                                           int HI, int L, int Lc, uint32_t* __restrict__ cbits,
                                                           int32_t* __restrict__ cpos, int nch) {
  constexpr int UNR = 4;
  constexpr int PER = IC / ST;
  __shared__ SelSmem sm;
  __shared__ __align__(16) uint32_t sb[IC];  // the chunk's score bits, position order
  const int b = blockIdx.y, c = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j = lane & 31, half = lane >> 5;
  IndexerQuery<DI, NT> Q;
  indexer_load_query<DI, NT>(Q, qI, w, b, HI, lane);
  const uint8_t* kb = kI + (int64_t)b * Lc * DI;
  float* Sb = S + (int64_t)b * L;
  const int p0 = c * IC;
  const int nv = min(IC, L - p0);
  for (int base = wave * 32 * UNR; base < nv; base += 4 * 32 * UNR) {
    float tot[UNR];
    indexer_round<DI, NT, UNR>(Q, kb, p0 + base, L, lane, tot);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int e = base + 32 * u + j;
      if (half == 0 && e < nv) {
        Sb[p0 + e] = tot[u];
        sb[e] = __float_as_uint(tot[u]);
      }
    }
  }
  __syncthreads();
  const int64_t slot0 = ((int64_t)b * nch + c) * IC_KEEP;
  if (nv <= IC_KEEP) {  // a short last chunk: every position is a candidate
    for (int e = t; e < nv; e += ST) {
      cbits[slot0 + e] = sb[e];
      cpos[slot0 + e] = p0 + e;
    }
    return;
  }
  uint32_t bits[PER], key[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(sb + t * PER + i);
    bits[i] = x.x; bits[i + 1] = x.y; bits[i + 2] = x.z; bits[i + 3] = x.w;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = score_key(__uint_as_float(bits[i]));
  uint32_t T, need_eq;
  block_kth_regs<PER>(key, nv, IC_KEEP, sm, &T, &need_eq);
  block_emit_regs<PER>(key, [&](int i) { return bits[i]; }, [&](int i) { return p0 + t * PER + i; }, nv, T, need_eq, sm, cpos + slot0,
                       reinterpret_cast<float*>(cbits + slot0));
}

// One workgroup of NW waves per sequence, PER candidates per thread in registers (candidate
// e = t * PER + i, chunk e / IC_KEEP). Dynamic LDS: the select's SelSmemT, or select_row_device's
// layout for the full-select path, which the first four waves run while the others leave (a
// workgroup barrier waits for the waves that have not ended). The indexer step (8192 candidates)
// took 0.049 ms with one 4-wave workgroup of 32 candidates a thread, 0.0435 with 8 waves of 16.
template <int PER, int NW>
__global__ __launch_bounds__(64 * NW) void indexer_finish_kernel(
    const float* __restrict__ S, int L, int k, const uint32_t* __restrict__ cbits, const int32_t* __restrict__ cpos,
    int nch, int ncand, int32_t* __restrict__ idx, float* __restrict__ sel, int capw) {
  static_assert(PER % IC_KEEP == 0 && PER % 4 == 0, "a thread holds whole chunks");
  static_assert(NW >= SW, "the full-select path runs on the first SW waves");
  constexpr int NT = 64 * NW;
  extern __shared__ uint4 smem_raw[];
  SelSmemT<NB0, NW>& sm = *reinterpret_cast<SelSmemT<NB0, NW>*>(smem_raw);
  const int b = blockIdx.x, t = threadIdx.x;
  const int kk = min(k, L);
  int32_t* oidx = idx + (int64_t)b * k;
  float* osel = sel ? sel + (int64_t)b * k : nullptr;
  bool full = ncand < kk;  // workgroup-uniform
  if (!full) {
    const uint32_t* gb = cbits + (int64_t)b * nch * IC_KEEP;
    const int32_t* gp = cpos + (int64_t)b * nch * IC_KEEP;
    const int e0 = t * PER;
    uint32_t bits[PER], key[PER];
    int32_t pos[PER];
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      if (e0 + i + 3 < ncand) {
        const uint4 x = ld16(gb + e0 + i), y = ld16(gp + e0 + i);
        bits[i] = x.x; bits[i + 1] = x.y; bits[i + 2] = x.z; bits[i + 3] = x.w;
        pos[i] = (int32_t)y.x; pos[i + 1] = (int32_t)y.y; pos[i + 2] = (int32_t)y.z; pos[i + 3] = (int32_t)y.w;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool in = e0 + i + u < ncand;
          bits[i + u] = in ? gb[e0 + i + u] : 0u;
          pos[i + u] = in ? gp[e0 + i + u] : -1;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = score_key(__uint_as_float(bits[i]));
    uint32_t T, need_eq;
    block_kth_regs<PER>(key, ncand, (uint32_t)kk, sm, &T, &need_eq);
    // a chunk with more positions than candidates whose smallest candidate key is >= T could hold
    // a kept position that is not a candidate
    bool risk = false;
#pragma unroll
    for (int cc = 0; cc < PER / IC_KEEP; ++cc) {
      const int c = (e0 + cc * IC_KEEP) / IC_KEEP;
      if (c < nch && min(IC, L - c * IC) > IC_KEEP) {
        uint32_t m = 0xffffffffu;
#pragma unroll
        for (int i = 0; i < IC_KEEP; ++i) m = min(m, key[cc * IC_KEEP + i]);
        risk |= m >= T;
      }
    }
    full = __syncthreads_or(risk) != 0;
    if (!full) {
      for (int jj = kk + t; jj < k; jj += NT) {
        oidx[jj] = -1;
        if (osel) osel[jj] = -INFINITY;
      }
      block_emit_regs<PER>(key, [&](int i) { return bits[i]; }, [&](int i) { return pos[i]; }, ncand, T, need_eq,
                           sm, oidx, osel);
      return;
    }
    __syncthreads();  // every wave is done with the select's LDS before the row select reuses it
  }
  if (t >= ST) return;  // whole waves (workgroup-uniform branch above): the row select takes SW waves
  select_row_device(S + (int64_t)b * L, L, L, k, kk, oidx, osel, capw, smem_raw);
}

constexpr int REGS_STAGE = 4096;  // most kept pairs the register select stages in LDS (32 KiB)

// Rows of at most 64 * NW * PER elements, held in registers by a workgroup of NW waves (thread t
// the elements t*PER ..): one load of the row, then the k' largest keys by relative-range
// histograms and the critical bin's few keys ranked one by one (block_kth_regs), and the kept
// elements emitted in position order with one block scan (block_emit_regs). The same selection as
// select_row_device: the k' largest keys, the lower position first among equal keys, positions
// ascending; -1 and -inf past k'.
template <int PER, int NW>
__global__ __launch_bounds__(64 * NW) void select_regs_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                              int k, int32_t* __restrict__ idx,
                                                              float* __restrict__ sel,
                                                              const int32_t* __restrict__ krow) {
  static_assert(PER % 4 == 0, "16-byte loads of a thread's run");
  constexpr int NT = 64 * NW;
  constexpr int STG = NT * PER < REGS_STAGE ? NT * PER : REGS_STAGE;  // kept pairs staged in LDS
  __shared__ SelSmemT<NB0, NW> sm;
  __shared__ uint32_t stg[2 * STG];  // kept positions, then their score bits
  const int64_t row = blockIdx.x;
  const float* s = S + row * stride;
  const int kk = max(0, min(krow ? min(krow[row], k) : k, n));  // krow: a count per row, at most k
  int32_t* oidx = idx + row * k;
  float* osel = sel ? sel + row * k : nullptr;
  const int t = threadIdx.x;
  for (int j = kk + t; j < k; j += NT) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  if (kk == 0) return;  // workgroup-uniform
  const int e0 = t * PER;
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  // only the keys stay in registers; a kept element's score bits come back from its key, except
  // for the keys that lose them (+-0, NaN), which are read again
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    uint32_t b[4];
    if (vec && e0 + i + 3 < n) {
      const uint4 x = ld16(s + e0 + i);
      b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = e0 + i + u < n ? __float_as_uint(s[e0 + i + u]) : 0u;
    }
    // elements past n take key 0 (a NaN's): they rank below every element and after every NaN of
    // the row (higher positions), and k' <= n never reaches them, so all NT * PER count as valid
    // and no per-element bound test is kept live
#pragma unroll
    for (int u = 0; u < 4; ++u) key[i + u] = e0 + i + u < n ? score_key(__uint_as_float(b[u])) : 0u;
  }
  auto bits_of = [&](int i) -> uint32_t {
    const uint32_t kx = key[i];
    if (kx == 0u || kx == 0x80000000u) return __float_as_uint(s[e0 + i]);
    return (kx & 0x80000000u) ? kx ^ 0x80000000u : ~kx;
  };
  uint32_t T, need_eq;
  block_kth_regs<PER>(key, NT * PER, (uint32_t)kk, sm, &T, &need_eq);
  if (kk <= STG) {  // the kept pairs staged in LDS and written out in whole lines
    block_emit_regs_staged<PER>(key, bits_of, [&](int i) { return e0 + i; }, NT * PER, T, need_eq, kk, sm, stg,
                                stg + STG, oidx, osel);
  } else {
    block_emit_regs<PER>(key, bits_of, [&](int i) { return e0 + i; }, NT * PER, T, need_eq, sm, oidx, osel);
  }
}

// A select of n <= REGS_NMAX elements per row goes through select_regs_kernel with one 256-thread
// workgroup per row. Measured on the two-level step's selects (1024 rows): 2048 -> 128 blocks in
// 9.4 us against about 15 for select_rows_kernel; 8192 -> 4096 candidates (32 per thread) in 35 us
// against 60 (64 when the kept pairs were written straight from registers, one scattered word per
// lane). A few rows (fewer than WIDE_ROWS) of up to WIDE_NMAX elements take 1024-thread
// workgroups instead: a row then needs no split over several workgroups and launches.
#ifndef TKA_REGS_NMAX
#define TKA_REGS_NMAX 8192
#endif
constexpr int REGS_NMAX = TKA_REGS_NMAX;
#ifndef TKA_WIDE_ROWS
#define TKA_WIDE_ROWS 128
#endif
#ifndef TKA_WIDE_NW
#define TKA_WIDE_NW 16
#endif
constexpr int WIDE_NMAX = 32768, WIDE_ROWS = TKA_WIDE_ROWS;
// waves of a wide workgroup: 16 (32 elements per thread) or 8 (64). Measured: 32 rows x 32768,
// k' = 2048 in 21.4 us with 16 waves (44 bytes per lane spilled at the 128-register cap) against
// 26.4 with 8 and 38.6 for the split select of several launches; the C2 step 0.0649 -> 0.048 ms
constexpr int WIDE_NW = TKA_WIDE_NW;

static void launch_select_regs(const SelectArgs& a, const int32_t* krow, hipStream_t st) {
  const dim3 grid((unsigned)a.n_rows), blk(ST);
  if (a.n <= 256 * 8)
    hipLaunchKernelGGL((select_regs_kernel<8, SW>), grid, blk, 0, st, a.scores, a.n, a.stride, a.k, a.idx, a.sel,
                       krow);
  else if (a.n <= 256 * 16)
    hipLaunchKernelGGL((select_regs_kernel<16, SW>), grid, blk, 0, st, a.scores, a.n, a.stride, a.k, a.idx, a.sel,
                       krow);
  else if (a.n <= REGS_NMAX)
    hipLaunchKernelGGL((select_regs_kernel<32, SW>), grid, blk, 0, st, a.scores, a.n, a.stride, a.k, a.idx, a.sel,
                       krow);
  else if (a.n <= 1024 * 16)
    hipLaunchKernelGGL((select_regs_kernel<16, 16>), grid, dim3(1024), 0, st, a.scores, a.n, a.stride, a.k, a.idx,
                       a.sel, krow);
  else  // n <= WIDE_NMAX
    hipLaunchKernelGGL((select_regs_kernel<WIDE_NMAX / (64 * WIDE_NW), WIDE_NW>), grid, dim3(64 * WIDE_NW), 0, st,
                       a.scores, a.n, a.stride, a.k, a.idx, a.sel, krow);
}

// ---------------------------------------------------------------------------
// Many long rows of a score array: the fused exact step's candidate select
// run over stored scores. 32 runs of 64 consecutive scores per row give each
// row a threshold T a few standard deviations below its k'-th score
// (prefilter_threshold_kernel, which also clears the row's count and flags);
// one pass over every row on the whole chip keeps the (score bits, position)
// pairs with key >= key(T) (rows_collect_kernel); prefilter_finish_kernel
// selects the k' first among them and flags the rows whose candidates cannot
// hold the answer (fewer than k', more than the capacity, a crowded tie bin),
// which select_rows_kernel then selects over the whole row.
// ---------------------------------------------------------------------------
constexpr int RC_RUNS = 32, RC_NSAMP = RC_RUNS * 64;
#ifndef TKA_RC_CHUNK
#define TKA_RC_CHUNK 32768
#endif
constexpr int RC_CHUNK = TKA_RC_CHUNK;  // positions per collect workgroup (two rounds)
constexpr int RC_ROUND = 16384;        // positions per round of it: 16 float4 loads per thread
static_assert(RC_CHUNK % RC_ROUND == 0, "whole rounds per chunk");

__global__ __launch_bounds__(256) void rows_sample_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                          float* __restrict__ samp) {
  const int64_t row = blockIdx.x;
  const float* s = S + row * stride;
  float v[RC_NSAMP / 256];
#pragma unroll
  for (int u = 0; u < RC_NSAMP / 256; ++u) {
    const int i = u * 256 + threadIdx.x, run = i >> 6;
    v[u] = s[(int64_t)run * n / RC_RUNS + (i & 63)];
  }
#pragma unroll
  for (int u = 0; u < RC_NSAMP / 256; ++u) samp[row * RC_NSAMP + u * 256 + threadIdx.x] = v[u];
}

constexpr int RC_STAGE = 1024;  // pairs a wave compacts in LDS before writing them out

// Kept: key(s) >= key(T), which for a number T is the float test s >= T (NaN scores fail it, -0
// equals +0), and everything when T is NaN. Each round is counted, reserved with one atomic per
// wave, and its kept pairs staged in LDS, which the wave copies out with full-width stores.
__global__ __launch_bounds__(256) void rows_collect_kernel(const float* __restrict__ S, int n, int64_t stride,
                                                           const float* __restrict__ Tv, uint2* __restrict__ cpair,
                                                           uint32_t* __restrict__ cnt, int capg) {
  constexpr int U = RC_ROUND / (256 * 4);
  __shared__ uint2 stage_all[SW][RC_STAGE];
  const int64_t row = blockIdx.y;
  const float* s = S + row * stride;
  const float Tf = Tv[row];
  const bool tnan = Tf != Tf;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  uint2* out = cpair + row * (int64_t)capg;
  uint2* stage = stage_all[w];
  const int c0 = blockIdx.x * RC_CHUNK, c1 = min(n, c0 + RC_CHUNK);
  for (int p0 = c0; p0 < c1; p0 += RC_ROUND) {
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = p0 + (u * 256 + (int)threadIdx.x) * 4;  // n is a multiple of 4: e < n covers all four
      uint4 r4 = make_uint4(0, 0, 0, 0);
      if (e < c1) r4 = ld16_stream(s + e);
      x[u] = make_float4(__uint_as_float(r4.x), __uint_as_float(r4.y), __uint_as_float(r4.z), __uint_as_float(r4.w));
    }
    auto kept = [&](int u, float v) {
      return p0 + (u * 256 + (int)threadIdx.x) * 4 < c1 && (tnan || v >= Tf);
    };
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      c += (kept(u, x[u].x) ? 1u : 0u) + (kept(u, x[u].y) ? 1u : 0u) + (kept(u, x[u].z) ? 1u : 0u) +
           (kept(u, x[u].w) ? 1u : 0u);
#pragma unroll
    for (int u = 0; u < U; ++u) {  // the tests are made again below, not held in scalar masks
      pin_vgpr(x[u].x);
      pin_vgpr(x[u].y);
      pin_vgpr(x[u].z);
      pin_vgpr(x[u].w);
    }
    // the wave's pairs of the round go to one reserved run of the row's list
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (tot == 0) continue;  // wave-uniform
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&cnt[row], tot);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
    uint32_t slot = incl - c;  // this lane's first pair within the wave's run
    if (tot <= (uint32_t)RC_STAGE) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = p0 + (u * 256 + (int)threadIdx.x) * 4;
        const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kept(u, v[j])) stage[slot++] = make_uint2(__float_as_uint(v[j]), (uint32_t)(e + j));
      }
      lds_wave_sync();
      for (uint32_t i = lane; i < tot && base + i < (uint32_t)capg; i += 64) out[base + i] = stage[i];
      lds_wave_sync();  // the stage's reads are done before the next round writes it
    } else {  // a crowded wave: direct stores
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = p0 + (u * 256 + (int)threadIdx.x) * 4;
        const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kept(u, v[j])) {
            if (base + slot < (uint32_t)capg) out[base + slot] = make_uint2(__float_as_uint(v[j]), (uint32_t)(e + j));
            ++slot;
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static bool use_split(int64_t n_rows, int n) { return n_rows < 128 && n > 4 * CHUNK; }

// the split finish keeps one offset per (chunk, wave) segment in LDS
bool select_len_supported(int64_t n_rows, int n) {
  return !use_split(n_rows, n) || sizeof(uint32_t) * (((size_t)n + CHUNK - 1) / CHUNK) * SW <= FIN_DYN_MAX;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SplitLayout {
  size_t ghist, cbits, cpos, ccount, catb, catp, total;
};

struct RowCandPlan {
  bool on = false;
  int r = 0, capg = 0;
};

// Rows the candidate select takes: many (the split mode takes few), long, k' <= n/8 and within the
// finish's limits, n a multiple of 4 (float4 loads; the row stride and base are checked at launch)
static RowCandPlan row_cand_plan(int64_t n_rows, int n, int k) {
  RowCandPlan pl;
  const int kk = std::min(k, n);
  if (use_split(n_rows, n) || n_rows < 64 || n < 16384 || n > 262144 || (n & 3) || kk < 1 || (int64_t)kk * 8 > n ||
      kk > PF_KMAX)
    return pl;
  const double E = (double)kk * RC_NSAMP / n;
  pl.r = std::min(RC_NSAMP, (int)std::ceil(E + 4.5 * std::sqrt(E)) + 2);
  const double expect = (double)n * (pl.r + 4.0 * std::sqrt((double)pl.r)) / RC_NSAMP;
  pl.capg = (int)std::max(3.0 * kk, std::ceil(expect));
  if (pl.capg > 12288) return RowCandPlan{};
  pl.on = true;
  return pl;
}

struct RowCandLayout {
  size_t samp, T, cnt, flag, gflag, cpair, total;
};

static RowCandLayout row_cand_layout(int64_t n_rows, const RowCandPlan& pl) {
  RowCandLayout L;
  size_t o = 0;
  L.samp = o; o += al256(sizeof(float) * (size_t)n_rows * RC_NSAMP);
  L.T = o; o += al256(sizeof(float) * (size_t)n_rows);
  L.cnt = o; o += al256(sizeof(uint32_t) * (size_t)n_rows);
  L.flag = o; o += al256(sizeof(uint32_t) * (size_t)n_rows);
  L.gflag = o; o += al256(sizeof(uint32_t) * (size_t)n_rows);
  L.cpair = o; o += al256(sizeof(uint2) * (size_t)n_rows * pl.capg);
  L.total = o;
  return L;
}

static SplitLayout split_layout(int64_t n_rows, int n) {
  const int64_t nch = (n + CHUNK - 1) / CHUNK;
  SplitLayout L;
  size_t o = 0;
  L.ghist = o; o += al256(sizeof(uint32_t) * n_rows * (NB0 + NB1));  // level 0 [rows][NB0], then level 1 [rows][NB1]
  L.cbits = o; o += al256(sizeof(uint32_t) * n_rows * (size_t)n);
  L.cpos = o; o += al256(sizeof(int32_t) * n_rows * (size_t)n);
  L.ccount = o; o += al256(sizeof(uint32_t) * n_rows * nch * SW);
  L.catb = o; o += al256(sizeof(uint32_t) * n_rows * (size_t)n);
  L.catp = o; o += al256(sizeof(int32_t) * n_rows * (size_t)n);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Certified adaptive k ("A Mathematical Theory of Top-k Sparse Attention via
// Total Variation Distance", abstract): the total-variation distance between
// a row's softmax P and its top-k truncation is the mass the truncation
// discards, so the smallest k with TV <= eps is the smallest prefix of the
// select order holding at least 1 - eps of the mass. Found by the same radix
// search over score keys, with histograms of mass next to the counts.
// Masses: w = exp(s - max) in fp32 (an element equal to the maximum: 1; NaN:
// 0), as floor(w * 2^40) in uint64, so every sum is exact and independent of
// the order of the atomics. The kept mass must reach need = W - floor(eps W)
// (W: the row total). Elements with the threshold key T all carry the same
// mass w_T, so after the keys above T the ties (lowest positions first, as in
// the select order) are taken ceil(rest / w_T) at a time. k is clamped to
// [max(k_min, 1), min(k_max, n)]; a row without mass keeps max(k_min, 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ak_mass(float v, float M) {
  if (v != v) return 0;
  const float w = (v == M) ? 1.f : expf(v - M);
  return (uint64_t)(w * 1099511627776.f);  // 2^40: exact scaling, the conversion truncates
}

// Radix levels of the adaptive search: 11, 11 and 10 bits of the key.
__device__ __forceinline__ int ak_shift(int lv) { return lv == 0 ? 21 : (lv == 1 ? 10 : 0); }
__device__ __forceinline__ int ak_bins(int lv) { return lv == 2 ? 1024 : 2048; }
__device__ __forceinline__ uint32_t ak_digit(uint32_t key, int lv) { return (key >> ak_shift(lv)) & (ak_bins(lv) - 1); }
__device__ __forceinline__ bool ak_in_range(uint32_t key, int lv, uint32_t prefix) {
  return lv == 0 || (key >> ak_shift(lv - 1)) == prefix;
}

// 28 KiB of histograms, so that four rows fit one CU. Levels 0 and 1: mass[2048] then
// cnt[2048]; level 2: mass[1024], cnt[1024], then a count histogram per wave [4][1024].
constexpr int AK_BUF = 3584;
struct AkSmem {
  uint64_t buf[AK_BUF];
  uint64_t wm[SW];
  uint32_t wc[SW];
  uint32_t wk[SW];
  uint32_t egt[SW], eeq[SW];  // per wave: keys above T, keys equal to T
  uint64_t res_mass;
  uint32_t res_bin, res_cnt;
};
__device__ __forceinline__ uint64_t* ak_mass_h(AkSmem& sm) { return sm.buf; }
__device__ __forceinline__ uint32_t* ak_cnt_h(AkSmem& sm, int lv) {
  return reinterpret_cast<uint32_t*>(sm.buf + (lv == 2 ? 1024 : 2048));
}
__device__ __forceinline__ uint32_t* ak_wave_h(AkSmem& sm, int w) {
  return reinterpret_cast<uint32_t*>(sm.buf + 1536) + w * 1024;
}
static_assert(1536 + SW * 1024 / 2 <= AK_BUF && 2048 + 2048 / 2 <= AK_BUF, "histogram views exceed the buffer");
constexpr int AK_UNR = 8;  // float4 loads in flight per lane in the streaming passes
constexpr int AK_EJ = 16;  // lane-strided elements per lane per round of the emission pass

// Sampled path of long rows: the keys >= T0 (T0 a sample quantile with about AKF_WANT keys above
// it) are collected while the row's mass is summed, and the search runs on them in LDS.
constexpr int AKF_WANT = 2048;  // expected candidates per row
constexpr int AKF_CAP = 4096;   // candidates per row held in LDS (AKF_CAP / SW per wave)
constexpr int AKF_NB = 1024;    // bins of the candidates' relative histogram
struct AkCand {
  uint32_t bits[AKF_CAP];     // score bits, per wave in position order
  uint16_t off[AKF_CAP];      // position minus the wave's segment start
  uint64_t hmass[AKF_NB];     // relative histogram: mass and count per bin
  uint32_t hcnt[AKF_NB];      // (then the critical bin's keys)
};
struct AkFast {
  SelSmem sel;
  uint32_t samp[SEL_SAMPLES];
};
union AkShared {
  AkSmem ak;
  AkFast f;
  AkCand c;
};
// reductions and results of the sampled path (outside the union)
struct AkRed {
  uint64_t wm[SW];
  uint32_t wc[SW];
  uint32_t wk[SW];
  uint32_t gt[SW], eq[SW], obase[SW], eqbase[SW];
  uint64_t res_mass;
  uint32_t res_bin, res_cnt, aux;
  uint32_t tkey, tcnt;
  uint64_t tmass;
};

// Bin b (of nb, bins ascending with the key) where the mass of the bins above
// it stays below need and reaching into b meets it. Writes the bin, the mass
// and the count of the bins above it to sm.res_*.
template <typename Sm>
__device__ void ak_find_bin(Sm& sm, const uint64_t* mass, const uint32_t* cnt, int nb, uint64_t need) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int per = nb / ST;
  uint64_t m = 0;
  uint32_t c = 0;
  for (int i = 0; i < per; ++i) {
    m += mass[t * per + i];
    c += cnt[t * per + i];
  }
  // inclusive prefix over threads (bins ascending), then the part above this thread's bins
  uint64_t im = m;
  uint32_t ic = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t ym = __shfl_up(im, o, kWave);
    const uint32_t yc = __shfl_up(ic, o, kWave);
    if (lane >= o) {
      im += ym;
      ic += yc;
    }
  }
  if (lane == 63) {
    sm.wm[w] = im;
    sm.wc[w] = ic;
  }
  __syncthreads();
  uint64_t tm = 0;
  uint32_t tc = 0;
  for (int i = 0; i < SW; ++i) {
    if (i < w) {
      im += sm.wm[i];
      ic += sm.wc[i];
    }
    tm += sm.wm[i];
    tc += sm.wc[i];
  }
  const uint64_t above = tm - im;
  uint32_t cabove = tc - ic;
  if (above < need && need <= above + m) {
    uint64_t acc = above;
    for (int i = per - 1; i >= 0; --i) {
      const int b = t * per + i;
      if (acc + mass[b] >= need) {
        sm.res_bin = (uint32_t)b;
        sm.res_mass = acc;
        sm.res_cnt = cabove;
        break;
      }
      acc += mass[b];
      cabove += cnt[b];
    }
  }
  __syncthreads();
}

// One workgroup per row; wave w streams its own segment [r0, r1) of the row
// (UNR float4 loads in flight per lane), as the count-based row select does.
// Given rmax (rslots partial maxima per row, written beside the scores by the
// scoring pass), the long-row path takes the row maximum from them instead of
// a pass over the row.
// Rows whose k is the unclamped budget answer emit their kept set here (every
// key above T, then the first `ties` keys equal to T in position order);
// rows held by k_min or k_max, or without mass, are flagged for the
// count-based row select with their k.
__global__ __launch_bounds__(256) void adaptive_k_kernel(const float* __restrict__ S, int n, int64_t stride, float eps,
                                                         int k_min, int k_max, int32_t* __restrict__ kout,
                                                         uint64_t* __restrict__ Wout, float* __restrict__ Mout,
                                                         int32_t* __restrict__ idx, float* __restrict__ sel,
                                                         uint32_t* __restrict__ row_flag,
                                                         const uint32_t* __restrict__ rmax, int rslots) {
  __shared__ AkShared shm;
  __shared__ AkRed fr;
  AkSmem& sm = shm.ak;
  const int64_t row = blockIdx.x;
  const float* s = S + row * stride;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const bool aligned = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  const int seg = ((n + 4 * SW - 1) / (4 * SW)) * 4;
  const int r0 = min(n, w * seg), r1 = min(n, r0 + seg);
  // 0. Long rows: two passes (the maximum; the mass total while the keys >= T0 are collected),
  // then the search among the candidates in LDS. The result is the one the digit search below
  // finds (the smallest k under the same integer masses), whenever the candidates hold the mass
  // to keep; otherwise (or on crowding, ties, no mass) the row goes the digit-search way.
  if (n >= SEL_SAMPLE_MIN_N && n <= SEL_SAMPLE_MAX_N && aligned && (n & 3) == 0 && (stride & 3) == 0) {
    AkFast& f = shm.f;
    const int ns = SEL_SAMPLES, nch = ns / 64;
    for (int c = w; c < nch; c += SW) {
      const int64_t at = (int64_t)c * n / nch;
      f.samp[c * 64 + lane] = score_key(s[at + lane]);
    }
    __syncthreads();
    const uint32_t rs = (uint32_t)max((int64_t)1, min((int64_t)ns, (int64_t)AKF_WANT * ns / n));
    radix_kth_t<SW>([&](uint32_t e) { return f.samp[((e >> 6) * SW + w) * 64 + (e & 63)]; }, (uint32_t)(ns / SW),
                    0, 0u, rs, f.sel);
    const uint32_t T0 = f.sel.res[0];
    __syncthreads();  // the samples are spent
    // the row maximum: from the partial maxima the scoring pass wrote beside the scores, else a
    // pass over the row (every load one float4 with no branch around it)
    uint32_t mk = 0;
    if (rmax) {
      for (int i = t; i < rslots; i += ST) mk = max(mk, rmax[row * rslots + i]);
    } else {
      for (int base = r0; base < r1; base += 256 * AK_UNR) {
        float4 x[AK_UNR];
#pragma unroll
        for (int u = 0; u < AK_UNR; ++u)
          x[u] = *reinterpret_cast<const float4*>(s + min(base + u * 256 + 4 * lane, r1 - 4));
#pragma unroll
        for (int u = 0; u < AK_UNR; ++u)
          if (base + u * 256 + 4 * lane < r1)
            mk = max(max(max(mk, score_key(x[u].x)), score_key(x[u].y)), max(score_key(x[u].z), score_key(x[u].w)));
      }
    }
    mk = wave_max_u32(mk);
    if (lane == 0) fr.wk[w] = mk;
    __syncthreads();
    mk = 0;
    for (int i = 0; i < SW; ++i) mk = max(mk, fr.wk[i]);
    if (mk != 0u) {  // workgroup-uniform; a row with no number has no mass (the digit-search way)
      const float M = key_value(mk);
      // the mass total and the candidates, in position order per wave
      AkCand& cd = shm.c;
      constexpr uint32_t capw = AKF_CAP / SW;
      uint32_t* cb = cd.bits + w * capw;
      uint16_t* co = cd.off + w * capw;
      uint64_t wl = 0;
      uint32_t cnt = 0;
      for (int base = r0; base < r1; base += 256 * AK_UNR) {
        float4 x[AK_UNR];
#pragma unroll
        for (int u = 0; u < AK_UNR; ++u)
          x[u] = *reinterpret_cast<const float4*>(s + min(base + u * 256 + 4 * lane, r1 - 4));
#pragma unroll
        for (int u = 0; u < AK_UNR; ++u) {
          const int p0 = base + u * 256 + 4 * lane;
          const bool valid = p0 < r1;  // whole float4s: r1 is a multiple of 4
          const float v[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
          bool fk[4];
          uint32_t before = 0, tot = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wl += valid ? ak_mass(v[j], M) : 0ull;
            fk[j] = valid && score_key(v[j]) >= T0;
            const uint64_t bl = ballot(fk[j]);
            before += count_below(bl);
            tot += __popcll(bl);
          }
          uint32_t slot = cnt + before;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (fk[j]) {
              if (slot < capw) {
                cb[slot] = __float_as_uint(v[j]);
                co[slot] = (uint16_t)(p0 + j - r0);
              }
              ++slot;
            }
          }
          cnt += tot;
        }
      }
      wl = wave_sum(wl);
      if (lane == 0) {
        fr.wm[w] = wl;
        fr.wc[w] = cnt;
      }
      __syncthreads();
      uint64_t W = 0;
      bool over = false;
      for (int i = 0; i < SW; ++i) {
        W += fr.wm[i];
        over |= fr.wc[i] > capw;
      }
      const double drop = floor((double)eps * (double)W);
      const uint64_t need = drop >= (double)W ? 0 : W - (uint64_t)drop;
      // the candidates' mass (all keys >= T0, when none was dropped)
      uint64_t cm = 0;
      if (!over)
        for (uint32_t e = lane; e < cnt; e += 64) cm += ak_mass(__uint_as_float(cb[e]), M);
      cm = wave_sum(cm);
      __syncthreads();
      if (lane == 0) fr.wm[w] = cm;
      __syncthreads();
      uint64_t CM = 0;
      for (int i = 0; i < SW; ++i) CM += fr.wm[i];
      if (!over && need > 0 && CM >= need) {  // workgroup-uniform: T >= T0, every key >= T is here
        // relative histogram of the candidates over [T0, max]: mass and count per bin
        const uint32_t span = mk - T0;
        const int shift = span >= (uint32_t)AKF_NB ? (32 - __clz(span)) - 10 : 0;  // span >> shift < AKF_NB
        for (int i = t; i < AKF_NB; i += ST) {
          cd.hmass[i] = 0;
          cd.hcnt[i] = 0;
        }
        __syncthreads();
        for (uint32_t e = lane; e < cnt; e += 64) {
          const float v = __uint_as_float(cb[e]);
          const uint32_t d = (score_key(v) - T0) >> shift;
          atomicAdd(&cd.hcnt[d], 1u);
          const uint64_t m = ak_mass(v, M);
          if (m) atomicAdd(reinterpret_cast<unsigned long long*>(&cd.hmass[d]), (unsigned long long)m);
        }
        __syncthreads();
        ak_find_bin(fr, cd.hmass, cd.hcnt, AKF_NB, need);
        const uint32_t bin = fr.res_bin, inbin = cd.hcnt[bin];
        const uint64_t m_above = fr.res_mass;
        const uint32_t c_above = fr.res_cnt;
        __syncthreads();
        if (inbin <= (uint32_t)AKF_NB) {  // workgroup-uniform; else heavy ties: the digit-search way
          // the critical bin's keys, then T: the key where the mass from the top reaches need
          uint32_t* stash = cd.hcnt;  // the counts are spent
          if (t == 0) fr.aux = 0u;
          __syncthreads();
          for (uint32_t e = lane; e < cnt; e += 64) {
            const uint32_t key = score_key(__uint_as_float(cb[e]));
            if (((key - T0) >> shift) == bin) stash[atomicAdd(&fr.aux, 1u)] = key;
          }
          __syncthreads();
          for (uint32_t i = t; i < inbin; i += ST) {
            const uint32_t v = stash[i];
            uint64_t gm = 0, em = 0;
            uint32_t gc = 0;
            for (uint32_t j = 0; j < inbin; ++j) {
              const uint32_t x = stash[j];
              const uint64_t m = ak_mass(key_value(x), M);
              gm += x > v ? m : 0ull;
              em += x == v ? m : 0ull;
              gc += x > v;
            }
            if (m_above + gm < need && need <= m_above + gm + em) {  // every such i writes the same
              fr.tkey = v;
              fr.tmass = m_above + gm;
              fr.tcnt = c_above + gc;
            }
          }
          __syncthreads();
          const uint32_t T = fr.tkey;
          const uint64_t m_gt = fr.tmass;
          const uint64_t wT = ak_mass(key_value(T), M);
          const uint32_t ties = (uint32_t)((need - m_gt + wT - 1) / wT);
          const int64_t k_eps = (int64_t)fr.tcnt + ties;
          const int64_t lo = k_min > 1 ? k_min : 1, hi = k_max < n ? k_max : n;
          int64_t k = k_eps < lo ? lo : k_eps;
          if (k > hi) k = hi;
          if (t == 0) {
            kout[row] = (int32_t)k;
            Wout[row] = W;
            Mout[row] = M;
            row_flag[row] = k == k_eps ? 0u : 1u;
          }
          if (k != k_eps) return;  // held by k_min or k_max: the count-based row select
          int32_t* oidx = idx + row * k_max;
          float* osel = sel ? sel + row * k_max : nullptr;
          for (int j = (int)k + t; j < k_max; j += ST) {
            oidx[j] = -1;
            if (osel) osel[j] = -INFINITY;
          }
          emit_segments([&](uint32_t e, uint32_t& bits, int32_t& pos) { bits = cb[e]; pos = r0 + (int)co[e]; }, cnt, T,
                        ties, fr, oidx, osel, (uint32_t)k);
          return;
        }
      }
    }
    __syncthreads();  // the union is handed to the digit search
  }
  // 1. the row maximum in the select order (NaN lowest)
  uint32_t mk = 0;
  for (int base = r0; base < r1; base += 256 * AK_UNR) {
    float v[AK_UNR][4];
#pragma unroll
    for (int u = 0; u < AK_UNR; ++u) load4(s, base + u * 256 + 4 * lane, r1, aligned, v[u]);
#pragma unroll
    for (int u = 0; u < AK_UNR; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (base + u * 256 + 4 * lane + j < r1) mk = max(mk, score_key(v[u][j]));
  }
  mk = wave_max_u32(mk);
  if (lane == 0) sm.wk[w] = mk;
  __syncthreads();
  mk = 0;
  for (int i = 0; i < SW; ++i) mk = max(mk, sm.wk[i]);
  const float M = mk ? key_value(mk) : __int_as_float(0x7fc00000);  // no number in the row: no mass
  // 2. digit by digit: mass and count histograms of the keys inside the current prefix
  uint64_t need = 0, W = 0, m_gt = 0;
  uint32_t c_gt = 0, prefix = 0;
  int64_t k_eps = 0;
  bool found = true;
  // the last level also counts, per wave, the keys above its range and its keys per digit (for
  // the emission's per-wave output bases)
  uint32_t* whist = ak_wave_h(sm, w);
  uint64_t* mass = ak_mass_h(sm);
  uint32_t wgt = 0;
  for (int lv = 0; lv <= 2; ++lv) {
    const int nb = ak_bins(lv);
    uint32_t* cnt = ak_cnt_h(sm, lv);
    for (int i = t; i < nb; i += ST) {
      mass[i] = 0;
      cnt[i] = 0;
    }
    if (lv == 2)
      for (int i = lane; i < 1024; i += 64) whist[i] = 0;
    __syncthreads();
    for (int base = r0; base < r1; base += 256 * AK_UNR) {
      float v[AK_UNR][4];
#pragma unroll
      for (int u = 0; u < AK_UNR; ++u) load4(s, base + u * 256 + 4 * lane, r1, aligned, v[u]);
#pragma unroll
      for (int u = 0; u < AK_UNR; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t key = score_key(v[u][j]);
          const bool valid = base + u * 256 + 4 * lane + j < r1;
          if (valid && ak_in_range(key, lv, prefix)) {
            const uint32_t d = ak_digit(key, lv);
            atomicAdd(&cnt[d], 1u);
            if (lv == 2) atomicAdd(&whist[d], 1u);
            const uint64_t m = ak_mass(v[u][j], M);
            if (m) atomicAdd(reinterpret_cast<unsigned long long*>(&mass[d]), (unsigned long long)m);
          } else if (lv == 2 && valid && (key >> ak_shift(1)) > prefix) {
            ++wgt;
          }
        }
    }
    __syncthreads();
    if (lv == 0) {
      uint64_t part = 0;
      for (int i = t; i < nb; i += ST) part += mass[i];
      part = wave_sum(part);
      if (lane == 0) sm.wm[w] = part;
      __syncthreads();
      for (int i = 0; i < SW; ++i) W += sm.wm[i];
      __syncthreads();
      const double drop = floor((double)eps * (double)W);
      need = drop >= (double)W ? 0 : W - (uint64_t)drop;
      if (need == 0) {
        found = false;  // nothing to keep for the budget
        break;
      }
    }
    ak_find_bin(sm, mass, cnt, nb, need - m_gt);
    m_gt += sm.res_mass;
    c_gt += sm.res_cnt;
    prefix = (prefix << (lv == 2 ? 10 : 11)) | sm.res_bin;
    __syncthreads();
  }
  uint32_t ties = 0;
  if (found) {  // the ties at T: ceil(rest / w_T) of them
    const uint64_t wT = ak_mass(key_value(prefix), M);
    const uint64_t rest = need - m_gt;
    ties = (uint32_t)((rest + wT - 1) / wT);
    k_eps = (int64_t)c_gt + ties;
  }
  const int64_t lo = k_min > 1 ? k_min : 1, hi = k_max < n ? k_max : n;
  int64_t k = k_eps < lo ? lo : k_eps;
  if (k > hi) k = hi;
  if (t == 0) {
    kout[row] = (int32_t)k;
    Wout[row] = W;
    Mout[row] = M;
  }
  const bool direct = found && k == k_eps;
  if (t == 0) row_flag[row] = direct ? 0u : 1u;
  if (!direct) return;  // workgroup-uniform
  // 3. emit: every key above T and the first `ties` keys equal to T, in position order. Wave w's
  // keys above T: those above the last level's range plus its digits above T's; equal: T's digit.
  int32_t* oidx = idx + row * k_max;
  float* osel = sel ? sel + row * k_max : nullptr;
  for (int j = (int)k + t; j < k_max; j += ST) {
    oidx[j] = -1;
    if (osel) osel[j] = -INFINITY;
  }
  const uint32_t T = prefix, dT = T & (NB1 - 1);
  {
    uint32_t g = 0;
    for (int i = lane; i < NB1; i += 64) g += (uint32_t)i > dT ? whist[i] : 0u;
    g = wave_sum(g) + wave_sum(wgt);
    if (lane == 0) {
      sm.egt[w] = g;
      sm.eeq[w] = whist[dT];
    }
  }
  __syncthreads();
  uint32_t run = 0, eqrun = 0;  // this wave's first output slot and first tie rank
  for (int i = 0; i < w; ++i) {
    const uint32_t take = ties > eqrun ? min(ties - eqrun, sm.eeq[i]) : 0u;
    run += sm.egt[i] + take;
    eqrun += sm.eeq[i];
  }
  // lane-strided rounds, so that a ballot over one element slot covers consecutive positions
  for (int base = r0; base < r1; base += 64 * AK_EJ) {
    float v[AK_EJ];
#pragma unroll
    for (int j = 0; j < AK_EJ; ++j) v[j] = s[min(base + 64 * j + lane, r1 - 1)];
#pragma unroll
    for (int j = 0; j < AK_EJ; ++j) {
      const int p = base + 64 * j + lane;
      const uint32_t key = score_key(v[j]);
      const bool valid = p < r1;
      const bool gt = valid && key > T;
      const bool eq = valid && key == T;
      const uint64_t be = ballot(eq);
      const bool take = gt || (eq && eqrun + (uint32_t)count_below(be) < ties);
      const uint64_t bs = ballot(take);
      const uint32_t slot = run + (uint32_t)count_below(bs);
      if (take && slot < (uint32_t)k) {  // exactly k keys are taken
        oidx[slot] = p;
        if (osel) osel[slot] = v[j];
      }
      run += (uint32_t)__popcll(bs);
      eqrun += (uint32_t)__popcll(be);
    }
  }
}

// tau = 1 - (mass of the kept positions) / W, the kept mass summed exactly.
__global__ __launch_bounds__(256) void adaptive_tau_kernel(const float* __restrict__ S, int64_t stride,
                                                           const int32_t* __restrict__ idx, int k_max,
                                                           const int32_t* __restrict__ kout,
                                                           const uint64_t* __restrict__ W,
                                                           const float* __restrict__ Mrow, float* __restrict__ tau) {
  __shared__ uint64_t part[SW];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const float M = Mrow[row];
  const int ke = kout[row];
  uint64_t kept = 0;
  for (int j = t; j < ke; j += ST) kept += ak_mass(S[row * stride + idx[row * k_max + j]], M);
  kept = wave_sum(kept);
  if (lane == 0) part[w] = kept;
  __syncthreads();
  if (t == 0) {
    uint64_t tot = 0;
    for (int i = 0; i < SW; ++i) tot += part[i];
    const uint64_t Wr = W[row];
    tau[row] = Wr ? (float)((double)(Wr - tot) / (double)Wr) : __int_as_float(0x7fc00000);
  }
}

size_t select_workspace_bytes(int64_t n_rows, int n, int k) {
  if (use_split(n_rows, n)) return split_layout(n_rows, n).total;
  const RowCandPlan pc = row_cand_plan(n_rows, n, k);
  return pc.on ? row_cand_layout(n_rows, pc).total : 0;
}

// Let a kernel take dynamic LDS up to the device limit minus its own static
// LDS (read from the code object, alignment padding included). A refused
// request is cleared so it cannot surface as a later launch error.
static void allow_dynamic_lds(const void* kernel, int limit) {
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, kernel) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  const int dyn = limit - (int)fa.sharedSizeBytes;
  if (dyn <= 0 || hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, dyn) != hipSuccess)
    (void)hipGetLastError();
}

static int max_lds_bytes() {
  static int cached[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 64 * 1024;
    }
    allow_dynamic_lds((const void*)select_rows_kernel, v);
    allow_dynamic_lds((const void*)prefilter_finish_kernel, v);
    cached[dev] = v;
  }
  return cached[dev];
}

int device_lds_limit() { return max_lds_bytes(); }

void ensure_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return;
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& e : done)
    if (e.first == kernel && e.second == dev) return;
  allow_dynamic_lds(kernel, max_lds_bytes());
  done.emplace_back(kernel, dev);
}

static int rows_capw(int n, int k, size_t* lds) {
  const int kk = k < n ? k : n;
  // candidates per wave: 1.5 k' + 64 over the waves, in multiples of 64, at most what lets two
  // workgroups share a CU's LDS
  const size_t head = (sizeof(SelSmem) + 15) & ~(size_t)15;
  const int lds_max = max_lds_bytes();
  const int two = (int)(((size_t)lds_max / 2 - head) / (SW * 8)) & ~63;
  int capw = (int)((((int64_t)kk + kk / 2 + 64 + SW - 1) / SW + 63) & ~(int64_t)63);
  capw = std::max(64, std::min(capw, std::max(64, two)));
  while (capw > 64 && head + (size_t)SW * capw * 8 > (size_t)lds_max) capw -= 64;
  *lds = head + (size_t)SW * capw * 8;
  return capw;
}

void launch_select_rows_counts(const SelectArgs& a, const int32_t* krow, hipStream_t st) {
  if (a.n_rows <= 0) return;
  if (a.n <= REGS_NMAX || (a.n_rows < WIDE_ROWS && a.n <= WIDE_NMAX)) {  // the whole row in registers
    launch_select_regs(a, krow, st);
    return;
  }
  size_t lds;
  const int capw = rows_capw(a.n, a.k, &lds);
  hipLaunchKernelGGL(select_rows_kernel, dim3((unsigned)a.n_rows), dim3(ST), lds, st, a.scores, a.n, a.stride, a.k,
                     a.idx, a.sel, capw, (const uint32_t*)nullptr, krow);
}

void launch_select_rows_flagged(const SelectArgs& a, const uint32_t* row_flag, const int32_t* krow, hipStream_t st) {
  if (a.n_rows <= 0) return;
  size_t lds;
  const int capw = rows_capw(a.n, a.k, &lds);
  hipLaunchKernelGGL(select_rows_kernel, dim3((unsigned)a.n_rows), dim3(ST), lds, st, a.scores, a.n, a.stride, a.k,
                     a.idx, a.sel, capw, row_flag, krow);
}

void launch_select_adaptive(const SelectArgs& a, float eps, int k_min, int32_t* kout, uint64_t* W, float* M,
                            uint32_t* row_flag, float* tau, hipStream_t st, const uint32_t* rmax, int rslots) {
  if (a.n_rows <= 0) return;
  const unsigned rows = (unsigned)a.n_rows;
  hipLaunchKernelGGL(adaptive_k_kernel, dim3(rows), dim3(ST), 0, st, a.scores, a.n, a.stride, eps, k_min, a.k, kout,
                     W, M, a.idx, a.sel, row_flag, rslots > 0 ? rmax : nullptr, rslots);
  // rows whose k is held by k_min / k_max or that have no mass: the count-based row select
  size_t lds;
  const int capw = rows_capw(a.n, a.k, &lds);
  hipLaunchKernelGGL(select_rows_kernel, dim3(rows), dim3(ST), lds, st, a.scores, a.n, a.stride, a.k, a.idx, a.sel,
                     capw, (const uint32_t*)row_flag, (const int32_t*)kout);
  hipLaunchKernelGGL(adaptive_tau_kernel, dim3(rows), dim3(ST), 0, st, a.scores, a.stride, a.idx, a.k,
                     (const int32_t*)kout, (const uint64_t*)W, (const float*)M, tau);
}

void launch_select(const SelectArgs& a, void* ws, hipStream_t st) {
  if (a.n_rows <= 0) return;
  if (a.n <= SH_NMAX && a.k <= SH_KMAX) {
    hipLaunchKernelGGL(select_short_kernel, dim3((unsigned)((a.n_rows + 3) / 4)), dim3(256), 0, st, a.scores,
                       a.n_rows, a.n, a.stride, a.k, a.idx, a.sel);
    return;
  }
  if (a.n_rows < WIDE_ROWS && a.n > REGS_NMAX && a.n <= WIDE_NMAX) {  // a few rows, each in one workgroup
    launch_select_regs(a, nullptr, st);
    return;
  }
  if (!use_split(a.n_rows, a.n)) {
    const RowCandPlan pc = row_cand_plan(a.n_rows, a.n, a.k);
    if (pc.on && ws && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && (a.stride & 3) == 0) {
      const RowCandLayout L = row_cand_layout(a.n_rows, pc);
      char* base = static_cast<char*>(ws);
      float* samp = reinterpret_cast<float*>(base + L.samp);
      float* T = reinterpret_cast<float*>(base + L.T);
      uint32_t* cnt = reinterpret_cast<uint32_t*>(base + L.cnt);
      uint32_t* flag = reinterpret_cast<uint32_t*>(base + L.flag);
      uint32_t* gflag = reinterpret_cast<uint32_t*>(base + L.gflag);
      uint2* cpair = reinterpret_cast<uint2*>(base + L.cpair);
      hipLaunchKernelGGL(rows_sample_kernel, dim3((unsigned)a.n_rows), dim3(256), 0, st, a.scores, a.n, a.stride,
                         samp);
      launch_prefilter_threshold(samp, a.n_rows, RC_NSAMP, pc.r, T, cnt, flag, gflag, 1, 1, 1, st);
      hipLaunchKernelGGL(rows_collect_kernel, dim3((unsigned)((a.n + RC_CHUNK - 1) / RC_CHUNK), (unsigned)a.n_rows),
                         dim3(256), 0, st, a.scores, a.n, a.stride, (const float*)T, cpair, cnt, pc.capg);
      launch_prefilter_finish(cpair, cnt, T, pc.capg, a.n_rows, a.n, a.k, 1, 1, 1, a.idx, a.sel, flag, gflag, st);
      launch_select_rows_flagged(a, flag, nullptr, st);  // rows whose candidates cannot hold the answer
      return;
    }
    if (a.n <= REGS_NMAX) {  // the whole row in registers
      launch_select_regs(a, nullptr, st);
      return;
    }
    size_t lds;
    const int capw = rows_capw(a.n, a.k, &lds);
    hipLaunchKernelGGL(select_rows_kernel, dim3((unsigned)a.n_rows), dim3(ST), lds, st, a.scores, a.n, a.stride,
                       a.k, a.idx, a.sel, capw, (const uint32_t*)nullptr, (const int32_t*)nullptr);
    return;
  }
  const SplitLayout L = split_layout(a.n_rows, a.n);
  char* base = static_cast<char*>(ws);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(base + L.ghist);
  uint32_t* ghist1 = ghist + a.n_rows * NB0;
  uint32_t* cbits = reinterpret_cast<uint32_t*>(base + L.cbits);
  int32_t* cpos = reinterpret_cast<int32_t*>(base + L.cpos);
  uint32_t* ccount = reinterpret_cast<uint32_t*>(base + L.ccount);
  uint32_t* catb = reinterpret_cast<uint32_t*>(base + L.catb);
  int32_t* catp = reinterpret_cast<int32_t*>(base + L.catp);
  const int nch = (a.n + CHUNK - 1) / CHUNK;
  const int64_t nh = a.n_rows * (NB0 + NB1);
  hipLaunchKernelGGL(select_zero_kernel, dim3((unsigned)((nh + 255) / 256 < 1024 ? (nh + 255) / 256 : 1024)),
                     dim3(256), 0, st, ghist, nh);
  hipLaunchKernelGGL(select_chunk_hist_kernel, dim3(nch, (unsigned)a.n_rows), dim3(ST), 0, st, a.scores, a.n,
                     a.stride, a.k, ghist);
  hipLaunchKernelGGL(select_chunk_hist1_kernel, dim3(nch, (unsigned)a.n_rows), dim3(ST), 0, st, a.scores, a.n,
                     a.stride, a.k, ghist, ghist1);
  hipLaunchKernelGGL(select_chunk_collect_kernel, dim3(nch, (unsigned)a.n_rows), dim3(ST), 0, st, a.scores, a.n,
                     a.stride, a.k, ghist, ghist1, cbits, cpos, ccount, nch);
  const size_t seg = sizeof(uint32_t) * (size_t)nch * SW;  // <= FIN_DYN_MAX: select_len_supported
  const int lcap = (int)std::min<size_t>(FIN_LDS_CAP, (FIN_DYN_MAX - seg) / 8);
  hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)a.n_rows), dim3(ST), seg + 8 * (size_t)lcap, st,
                     a.scores, a.n, a.stride, a.k, ghist, ghist1, cbits, cpos, ccount, catb, catp, nch, a.idx,
                     a.sel, lcap);
}

void launch_prefilter_threshold(const float* samp, int64_t n_rows, int nsamp, int r, float* T, uint32_t* cnt,
                                uint32_t* row_flag, uint32_t* group_flag, int G, int Hq, int M, hipStream_t st) {
  if (n_rows <= 0) return;
  const dim3 grid((unsigned)((n_rows + 3) / 4));
  if (nsamp <= 2048)
    hipLaunchKernelGGL(prefilter_threshold_kernel<32>, grid, dim3(256), 0, st, samp, nsamp, r, n_rows, T, cnt,
                       row_flag, group_flag, G, Hq, M);
  else if (nsamp <= 4096)
    hipLaunchKernelGGL(prefilter_threshold_kernel<64>, grid, dim3(256), 0, st, samp, nsamp, r, n_rows, T, cnt,
                       row_flag, group_flag, G, Hq, M);
  else  // the plan keeps nsamp <= 8192
    hipLaunchKernelGGL(prefilter_threshold_kernel<128>, grid, dim3(256), 0, st, samp, nsamp, r, n_rows, T, cnt,
                       row_flag, group_flag, G, Hq, M);
}

int repair_slots(int64_t n_groups, int rows_per_group, int L) {
  // slots of 16 score rows within PF_REPAIR_BYTES (at least one, at most one per group, and enough
  // that no workgroup holds more than 256 groups)
  const int64_t per = (int64_t)std::min(16, rows_per_group) * L * (int64_t)sizeof(float);
  int64_t ns = std::max<int64_t>(1, (int64_t)PF_REPAIR_BYTES / std::max<int64_t>(per, 1));
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, n_groups));
  ns = std::max<int64_t>(ns, (n_groups + 255) / 256);
  return (int)ns;
}

size_t repair_slot_bytes(int64_t n_groups, int rows_per_group, int L) {
  return (size_t)repair_slots(n_groups, rows_per_group, L) * std::min(16, rows_per_group) * (size_t)L * sizeof(float);
}

template <int D>
static void launch_repair_d(const RepairArgs& a, hipStream_t st) {
  const int nslot = repair_slots((int64_t)a.B * a.Hkv, a.M * a.G, a.L);
  size_t sel_lds;
  const int capw = rows_capw(a.L, a.k, &sel_lds);
  const size_t lds = std::max(sel_lds, (size_t)4 * 32 * (D * 2 + 16));
  ensure_dynamic_lds((const void*)prefilter_repair_kernel<D>, lds);
  hipLaunchKernelGGL((prefilter_repair_kernel<D>), dim3((unsigned)nslot), dim3(ST), lds, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.K, a.Hq, a.Hkv, a.G, a.M, a.L, a.sb, a.sh, a.sl, a.scale, a.k,
                     a.B * a.Hkv, a.group_flag, a.row_flag, a.slots, a.idx, a.sel, capw);
}

void launch_prefilter_repair(const RepairArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: launch_repair_d<64>(a, st); break;
    case 128: launch_repair_d<128>(a, st); break;
    default: launch_repair_d<256>(a, st); break;
  }
}

// kept bitmap and prefix counts, ceil(n/32) words each, rounded up to whole 16-byte quads
static size_t prefilter_finish_lds(int n) { return sizeof(uint32_t) * 2 * (size_t)((((n + 31) / 32) + 3) & ~3); }

void launch_prefilter_finish(const uint2* cpair, const uint32_t* cnt, const float* T,
                             int capg, int64_t n_rows, int n, int k, int G, int Hq, int M, int32_t* idx, float* sel,
                             uint32_t* row_flag, uint32_t* group_flag, hipStream_t st) {
  (void)max_lds_bytes();
  hipLaunchKernelGGL(prefilter_finish_kernel, dim3((unsigned)n_rows), dim3(PF_T), prefilter_finish_lds(n), st, cpair,
                     cnt, T, capg, n, k, G, Hq, M, idx, sel, row_flag, group_flag);
}


IndexerCandPlan indexer_cand_plan(int L, int k) {
  IndexerCandPlan pl;
  pl.nch = (L + IC - 1) / IC;
  pl.ncand = pl.nch > 0 ? (pl.nch - 1) * IC_KEEP + std::min(IC_KEEP, L - (pl.nch - 1) * IC) : 0;
  // long rows only, at most four kept positions expected per chunk (k * IC <= 4 L: a chunk with more
  // than IC_KEEP of them is then far in the tail), and the candidates within the finish's LDS
  const int kk = std::min(k, L);
  pl.on = L >= 8 * IC && kk >= 1 && (int64_t)kk * IC <= 4 * (int64_t)L && pl.ncand <= IC_CAND_MAX && pl.ncand >= kk;
  return pl;
}

size_t indexer_cand_bytes(int64_t B, const IndexerCandPlan& pl) {
  return pl.on ? 2 * al256(sizeof(uint32_t) * (size_t)B * pl.nch * IC_KEEP) : 0;
}

template <int DI, int NT>
static void launch_icand_t(const IndexerArgs& a, const IndexerCandPlan& pl, uint32_t* cbits, int32_t* cpos,
                           hipStream_t st) {
  hipLaunchKernelGGL((indexer_cand_kernel<DI, NT>), dim3((unsigned)pl.nch, (unsigned)a.B), dim3(ST), 0, st, a.qI,
                     a.kI, a.w, a.scores, a.HI, a.L, a.Lc > 0 ? a.Lc : a.L, cbits, cpos, pl.nch);
}

template <int DI>
static void launch_icand_d(const IndexerArgs& a, const IndexerCandPlan& pl, uint32_t* cbits, int32_t* cpos,
                           hipStream_t st) {
  if (a.HI <= 32) launch_icand_t<DI, 1>(a, pl, cbits, cpos, st);
  else if (a.HI <= 64) launch_icand_t<DI, 2>(a, pl, cbits, cpos, st);
  else launch_icand_t<DI, 4>(a, pl, cbits, cpos, st);
}

void launch_indexer_select(const IndexerArgs& a, const IndexerCandPlan& pl, int k, void* cand_ws, int32_t* idx,
                           float* sel, hipStream_t st) {
  if (a.B <= 0) return;
  uint32_t* cbits = static_cast<uint32_t*>(cand_ws);
  int32_t* cpos = reinterpret_cast<int32_t*>(static_cast<char*>(cand_ws) +
                                             al256(sizeof(uint32_t) * (size_t)a.B * pl.nch * IC_KEEP));
  if (a.dI == 64) launch_icand_d<64>(a, pl, cbits, cpos, st);
  else launch_icand_d<128>(a, pl, cbits, cpos, st);
  size_t lds;
  const int capw = rows_capw(a.L, k, &lds);
  constexpr int FNW = 8;  // waves of the finish
  const size_t own = sizeof(SelSmemT<NB0, FNW>);
  if (lds < own) lds = own;
  auto go = [&](const void* kern, auto f) {
    ensure_dynamic_lds(kern, lds);
    f();
  };
  if (pl.ncand <= 16 * 64 * FNW)
    go((const void*)indexer_finish_kernel<16, FNW>, [&] {
      hipLaunchKernelGGL((indexer_finish_kernel<16, FNW>), dim3((unsigned)a.B), dim3(64 * FNW), lds, st, a.scores,
                         a.L, k, cbits, cpos, pl.nch, pl.ncand, idx, sel, capw);
    });
  else  // the plan keeps ncand <= IC_CAND_MAX = 32 * 64 * FNW
    go((const void*)indexer_finish_kernel<32, FNW>, [&] {
      hipLaunchKernelGGL((indexer_finish_kernel<32, FNW>), dim3((unsigned)a.B), dim3(64 * FNW), lds, st, a.scores,
                         a.L, k, cbits, cpos, pl.nch, pl.ncand, idx, sel, capw);
    });
}

}  // namespace tka
