// Two-level (hierarchical) selection for gfx950: "Sparse Attention
// Landscape", "Hierarchical Sparse Attention". The coarse level (block
// scores from the block means, top-K_B blocks) runs on the scoring and
// select kernels; here are the fine level's pieces: the exact scores of the
// kept blocks' tokens only, and the map from candidate slots back to
// positions.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace tka {

// One row (b, query head) per logical grid row; a workgroup takes bpw of its
// K_B kept blocks. Workgroup ids are remapped so that the rows of one KV
// group (which often keep the same blocks) run on one XCD and share its L2.
// Candidate slot t = j*bsz + i is token blk[j]*bsz + i; its score
// scale * <q, K_token> goes to cand[row, t], NaN where there is no token
// (blk[j] = -1 or past L). A lane group of LPR lanes holds one key row
// (16 bytes per lane), RPW rows per wave load, UNR loads in flight. The first
// workgroup of a row also writes krow[row] = min(k, the row's token count).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void hisa_token_score_kernel(const void* __restrict__ qv, const void* __restrict__ Kv,
                                                               const int32_t* __restrict__ blk, int KB, int bsz,
                                                               int Hq, int G, int L, int64_t sb, int64_t sh,
                                                               int64_t sl, float scale, int bpw, int k,
                                                               float* __restrict__ cand, int32_t* __restrict__ krow) {
  using U = Unpack<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = U::N;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int UNR = 4;
  // logical (row, block slice): the rows of one KV group are adjacent, so they share an XCD
  const unsigned lid = xcd_logical_id(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int64_t row = lid / gridDim.x;
  const unsigned bx = lid % gridDim.x;
  const int b = (int)(row / Hq), h = (int)(row % Hq), g = h / G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, grp = lane / LPR;
  const int32_t* lb = blk + row * KB;
  const int64_t ncand = (int64_t)KB * bsz;
  float* crow = cand + row * ncand;
  if (bx == 0 && threadIdx.x == 0) {
    int64_t n = 0;
    for (int j = 0; j < KB; ++j)
      if (lb[j] >= 0) n += min((int64_t)bsz, (int64_t)L - (int64_t)lb[j] * bsz);
    krow[row] = (int32_t)min((int64_t)k, n);
  }
  float qf[EPL];
  U::run(ld16(reinterpret_cast<const uint8_t*>(qv) + (row * D + sub * EPL) * ES), qf);
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(Kv) + ((int64_t)b * sb + (int64_t)g * sh) * ES;
  const int64_t t0 = (int64_t)bx * bpw * bsz, t1 = min(t0 + (int64_t)bpw * bsz, ncand);
  for (int64_t base = t0 + wave * RPW * UNR; base < t1; base += 4 * RPW * UNR) {
    uint4 raw[UNR];
    int pos[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t t = base + u * RPW + grp;
      int p = -1;
      if (t < t1) {
        const int j = lb[t / bsz];
        if (j >= 0) {
          const int64_t x = (int64_t)j * bsz + t % bsz;
          if (x < L) p = (int)x;
        }
      }
      pos[u] = p;
      raw[u] = p >= 0 ? ld16_stream(Kb + ((int64_t)p * sl + sub * EPL) * ES) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[EPL];
      U::run(raw[u], kf);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(qf[e], kf[e], a);
      a = group_sum<LPR>(a);
      const int64_t t = base + u * RPW + grp;
      if (t < t1 && sub == 0) crow[t] = pos[u] >= 0 ? a * scale : __int_as_float(0x7fc00000);
    }
  }
}

// The same candidate scores per KV group: the G query heads of a group keep
// overlapping blocks, so each block of the union of their kept lists is read
// once and scored for all G heads with v_mfma_f32_16x16x32_bf16 (16 keys x
// 16 head columns per tile; fragments loaded straight from K). A workgroup
// takes CB union blocks of one group. It first rebuilds the union in LDS: a
// bitmap over the m blocks and a popcount prefix per word, so union rank r
// gives block u. A head keeps u at slot j of its own list, found by binary
// search in its LDS copy of the list, and the tile's scores go to slots
// j*bsz + i. The first workgroup of a group also writes each row's count k'
// and NaN into the slots of list entries that are -1 (positions past L are NaN
// as above). Dynamic LDS: G*KB list words, then 2*ceil(m/32) bitmap and
// prefix words.
constexpr int HG_CB = 16;  // union blocks per workgroup
#ifndef TKA_HISA_GROUP
#define TKA_HISA_GROUP 1
#endif

template <int D>
__global__ __launch_bounds__(256) void hisa_group_score_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ K,
                                                               const int32_t* __restrict__ blk, int KB, int bsz,
                                                               int Hq, int G, int L, int m, int64_t sb, int64_t sh,
                                                               int64_t sl, float scale, int k, float* __restrict__ cand,
                                                               int32_t* __restrict__ krow) {
  constexpr int KS = D / 32;
  extern __shared__ int32_t hg_lds[];
  const int Hkv = Hq / G;
  const int task = blockIdx.y;  // (b, KV head)
  const int b = task / Hkv, g = task % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int64_t row0 = (int64_t)b * Hq + g * G;
  const int64_t ncand = (int64_t)KB * bsz;
  const int W = (m + 31) >> 5;
  int32_t* lists = hg_lds;                                       // [G][KB]
  uint32_t* bm = reinterpret_cast<uint32_t*>(hg_lds + G * KB);  // [W] union bitmap
  uint32_t* pre = bm + W;                                        // [W] set bits before each word
  __shared__ uint32_t part[4];
  for (int i = tid; i < G * KB; i += 256) lists[i] = blk[row0 * KB + i];
  for (int i = tid; i < W; i += 256) bm[i] = 0u;
  __syncthreads();
  for (int i = tid; i < G * KB; i += 256) {
    const int u = lists[i];
    if (u >= 0 && u < m) atomicOr(&bm[u >> 5], 1u << (u & 31));
  }
  __syncthreads();
  // exclusive popcount prefix over the words: thread t takes a contiguous run of them
  const int per = (W + 255) / 256;
  uint32_t loc = 0;
  for (int i = tid * per; i < min(W, tid * per + per); ++i) loc += __popc(bm[i]);
  const uint32_t incl = wave_incl_scan(loc);
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  uint32_t run = incl - loc, U = 0;
  for (int i = 0; i < 4; ++i) {
    run += i < wave ? part[i] : 0u;
    U += part[i];
  }
  for (int i = tid * per; i < min(W, tid * per + per); ++i) {
    pre[i] = run;
    run += __popc(bm[i]);
  }
  __syncthreads();
  if (blockIdx.x == 0) {  // counts, and NaN for the slots of -1 entries
    for (int h = wave; h < G; h += 4) {
      const int32_t* lh = lists + h * KB;
      int64_t nt = 0;
      for (int j = lane; j < KB; j += 64) {
        const int u = lh[j];
        if (u >= 0) nt += min((int64_t)bsz, (int64_t)L - (int64_t)u * bsz);
      }
      nt = wave_sum(nt);
      if (lane == 0) krow[row0 + h] = (int32_t)min((int64_t)k, nt);
      float* cr = cand + (row0 + h) * ncand;
      for (int j = 0; j < KB; ++j)
        if (lh[j] < 0)
          for (int i = lane; i < bsz; i += 64) cr[(int64_t)j * bsz + i] = __int_as_float(0x7fc00000);
    }
  }
  const uint32_t r0 = blockIdx.x * HG_CB;
  if (r0 >= U) return;  // workgroup-uniform
  // this workgroup's union blocks (ranks r0 .. r0 + HG_CB - 1) and each head's slot of them, found
  // once here, in parallel (a search per block and per (block, head)), rather than by every wave
  // in a dependent chain ahead of each block's loads
  __shared__ int32_t ublk[HG_CB];
  __shared__ int32_t uslot[HG_CB][16];
  if (tid < HG_CB && r0 + tid < U) {  // union rank r -> block u: the word holding it, then the bit
    const uint32_t r = r0 + tid;
    int lo = 0, hi = W - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    uint32_t x = bm[lo];
    for (uint32_t c = r - pre[lo]; c > 0; --c) x &= x - 1u;
    ublk[tid] = lo * 32 + __builtin_ctz(x);
  }
  __syncthreads();
  if (tid < HG_CB * G && r0 + tid / G < U) {  // head h's slot of block u (-1: not kept by head h)
    const int rr = tid / G, h = tid % G, u = ublk[rr];
    const int32_t* lh = lists + h * KB;
    int a = 0, z = KB - 1;
    while (a < z) {  // first entry >= u (-1 entries sit at the end and count as above every block)
      const int mid = (a + z) >> 1;
      const int v = lh[mid];
      if (v >= 0 && v < u) a = mid + 1;
      else z = mid;
    }
    uslot[rr][h] = lh[a] == u ? a : -1;
  }
  __syncthreads();
  // the G heads' query fragments (column n = head n)
  bf16x8_t bq[KS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q + (row0 + (n < G ? n : 0)) * D + 8 * kg);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const uint4 x = qp[4 * s2];
      bq[s2] = __builtin_bit_cast(bf16x8_t, n < G ? x : make_uint4(0, 0, 0, 0));
    }
  }
  const uint16_t* Kb = K + (int64_t)b * sb + (int64_t)g * sh;
  for (uint32_t r = r0 + wave; r < min(U, r0 + HG_CB); r += 4) {
    const int u = ublk[r - r0];
    const int j = n < G ? uslot[r - r0][n] : -1;  // head n's slot of block u
    const int p0 = u * bsz, pe = min(p0 + bsz, L);
    float* crow = j >= 0 ? cand + (row0 + n) * ncand + (int64_t)j * bsz : nullptr;
    for (int t0 = 0; t0 < bsz; t0 += 64) {  // up to four 16-key tiles at a time
      uint4 a[4][KS];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int pos = min(p0 + t0 + 16 * tt + n, pe - 1);
        const uint16_t* rp = Kb + (int64_t)pos * sl + 8 * kg;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) a[tt][s2] = (t0 + 16 * tt < bsz) ? ld16(rp + 32 * s2) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (t0 + 16 * tt >= bsz) break;  // wave-uniform
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[tt][s2]), bq[s2], acc, 0, 0, 0);
        if (crow) {
          const int e = t0 + 16 * tt + 4 * kg;  // slot offset inside the block
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = p0 + e + i < L ? acc[i] * scale : __int_as_float(0x7fc00000);
          *reinterpret_cast<float4*>(crow + e) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

template <int D>
static bool launch_hisa_group(const HisaArgs& a, hipStream_t st) {
  const int m = (a.L + a.bsz - 1) / a.bsz;
  const int W = (m + 31) / 32;
  const size_t lds = sizeof(int32_t) * ((size_t)a.G * a.KB + 2 * (size_t)W);
  if (lds > 64 * 1024) return false;
  const int umax = std::min(m, a.G * a.KB);
  const dim3 grid((unsigned)((umax + HG_CB - 1) / HG_CB), (unsigned)(a.B * (a.Hq / a.G)));
  hipLaunchKernelGGL((hisa_group_score_kernel<D>), grid, dim3(256), lds, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.K, a.blk, a.KB, a.bsz, a.Hq, a.G, a.L, m, a.sb, a.sh, a.sl, a.scale, a.k,
                     a.cand, a.krow);
  return true;
}

// Candidate slots (ascending, -1 padded) -> token positions, in place.
__global__ void hisa_map_kernel(int32_t* __restrict__ idx, const int32_t* __restrict__ blk, int64_t n, int k, int KB,
                                int bsz) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int s = idx[i];
    if (s >= 0) idx[i] = blk[(i / k) * KB + s / bsz] * bsz + s % bsz;
  }
}

template <bool BF16, int D>
static void launch_hisa_t(const HisaArgs& a, hipStream_t st) {
  const int bpw = 8;
  dim3 grid((a.KB + bpw - 1) / bpw, (unsigned)((int64_t)a.B * a.Hq));
  hipLaunchKernelGGL((hisa_token_score_kernel<BF16, D>), grid, dim3(256), 0, st, a.q, a.K, a.blk, a.KB, a.bsz, a.Hq,
                     a.G, a.L, a.sb, a.sh, a.sl, a.scale, bpw, a.k, a.cand, a.krow);
}

template <bool BF16>
static void launch_hisa_b(const HisaArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: launch_hisa_t<BF16, 64>(a, st); break;
    case 128: launch_hisa_t<BF16, 128>(a, st); break;
    default: launch_hisa_t<BF16, 256>(a, st); break;
  }
}

void launch_hisa_token_scores(const HisaArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.Hq <= 0 || a.KB <= 0) return;
  // bf16 groups of 2..16 heads, blocks of whole 16-key tiles: the per-group MFMA form
  if (a.bf16 && a.G >= 2 && a.G <= 16 && a.bsz % 16 == 0 && TKA_HISA_GROUP) {
    bool done = false;
    switch (a.d) {
      case 64: done = launch_hisa_group<64>(a, st); break;
      case 128: done = launch_hisa_group<128>(a, st); break;
      default: done = launch_hisa_group<256>(a, st); break;
    }
    if (done) return;
  }
  if (a.bf16) launch_hisa_b<true>(a, st);
  else launch_hisa_b<false>(a, st);
}

void launch_hisa_map(int32_t* idx, const int32_t* blk, int64_t rows, int k, int KB, int bsz, hipStream_t st) {
  const int64_t n = rows * k;
  if (n <= 0) return;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(hisa_map_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, st, idx, blk, n,
                     k, KB, bsz);
}

}  // namespace tka
