// Scoring kernels for gfx950.
//
// Exact token scores ("Sparse Attention Landscape", "Token Sparse Attention":
// s_i = f(q_t, k_i), here scale * <q, k_i>), block-mean scores (same page,
// "Block Sparse Attention": dot product of q with the mean-pooled keys of a
// block) and lightning-indexer scores (same page, "Token Sparse Attention":
// sum over indexer heads of w_j * ReLU(<q^I_j, k^I_i>)).
//
// All three stream their key rows once from HBM with 128-bit loads. The scan
// is bandwidth-bound (about G flop per byte for grouped heads), so MFMA is
// used only where several query heads share a key row (a real small-M
// contraction) and for the fp8 indexer; the rest uses wave dot-reductions.
#include "device_common.h"
#include "indexer_core.h"
#include "internal.h"

namespace tka {

// ---------------------------------------------------------------------------
// Exact scores, bf16, 2 <= G <= 16 query heads per KV head: one
// v_mfma_f32_16x16x32_bf16 tile = 16 positions x 16 heads (G used) x 32 dims.
// A = 16 key rows (lane l: row l%16, dims 8*(l/16)+[0,8) of each 32-dim step),
// B = q^T of the group (lane l: head l%16, same dims), C[pos][head]: lane l
// holds head l%16 for positions 4*(l/16)+[0,4). A position always sits in
// lane row pos%16 and the dims are summed in one fixed order, so every mode
// below produces bit-identical scores.
// Grid (chunks, B*Hkv), 256 threads; each wave takes 64 positions per round.
//   MFMA_FULL    - write every score, [B*Hq, L].
//   MFMA_SAMPLE  - only the first 64 positions of every chunk; wave w of
//                  workgroup x takes chunk 4x+w; scores to [B*Hq, nsamp].
// ---------------------------------------------------------------------------
enum { MFMA_FULL = 0, MFMA_SAMPLE = 1 };
// How K reaches the MFMA operand registers:
//   KLOAD_DIRECT    - each lane loads its own operand slice (16 rows x 64 B per
//                     load instruction), non-temporal.
//   KLOAD_DIRECT_RT - the same with ordinary (cached) loads.
//   KLOAD_STAGED    - fully coalesced non-temporal loads (every instruction
//                     reads whole rows, 1 KiB contiguous per wave) into a
//                     wave-private LDS area whose rows are padded by 16 B, then
//                     operand reads from LDS without bank conflicts.
enum { KLOAD_DIRECT = 0, KLOAD_DIRECT_RT = 1, KLOAD_STAGED = 2 };
#ifndef TKA_SCAN_KLOAD
#define TKA_SCAN_KLOAD KLOAD_STAGED
#endif

template <int D, int MODE, int KL>
__global__ __launch_bounds__(256) void score_exact_mfma_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ K, int Hq, int Hkv, int G,
                                                               int L, int64_t sb, int64_t sh, int64_t sl, float scale,
                                                               int chunk, MfmaOut o) {
  constexpr int KS = D / 32;
  constexpr int TILES = KL == KLOAD_STAGED ? 2 : 4;  // 16-position tiles per wave round
  constexpr int P = 16 * TILES;
  constexpr int RB = D * 2;              // bytes of a key row
  constexpr int PADB = RB + 16;          // LDS row stride
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;         // rows per coalesced load instruction
  constexpr int NI = KL == KLOAD_STAGED ? P / RPI : TILES * KS;  // load instructions per round
  const int task = blockIdx.y;
  const int b = task / Hkv, g = task % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int64_t row = (int64_t)b * Hq + g * G + (n < G ? n : 0);

  // dynamic LDS: staging rows, 4 waves x P rows x PADB
  extern __shared__ uint4 smem_raw[];
  uint8_t* stage_rows = reinterpret_cast<uint8_t*>(smem_raw) + (size_t)wave * P * PADB;

  bf16x8_t bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < G) v = ld16(q + ((int64_t)(b * Hq + g * G + n)) * D + 32 * s + 8 * kg);
    bq[s] = __builtin_bit_cast(bf16x8_t, v);
  }
  const uint16_t* Kb = K + (int64_t)b * sb + (int64_t)g * sh;
  int p0, p1, base, step;
  if (MODE == MFMA_SAMPLE) {
    const int c = blockIdx.x * 4 + wave;
    p0 = c * chunk;
    p1 = min(p0 + 64, L);
    base = p0;
    step = P;
  } else {
    p0 = blockIdx.x * chunk;
    p1 = min(p0 + chunk, L);
    base = p0 + wave * P;
    step = 4 * P;
  }
  const bool vec_store = (L & 3) == 0;

  auto load = [&](uint4 (&a)[NI], int at) {
    if (KL == KLOAD_STAGED) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int pos = min(at + j * RPI + lane / CPR, L - 1);
        a[j] = ld16_stream(Kb + (int64_t)pos * sl + (lane % CPR) * 8);
      }
    } else {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int pos = min(at + 16 * t + n, L - 1);
        const uint16_t* rp = Kb + (int64_t)pos * sl + 8 * kg;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          a[t * KS + s] = KL == KLOAD_DIRECT ? ld16_stream(rp + 32 * s) : ld16(rp + 32 * s);
      }
    }
  };

  uint4 cur[NI];
  uint32_t kmax = 0;  // full mode: the largest score key this lane wrote (head n)
  if (base < p1) load(cur, base);
  for (; base < p1; base += step) {
    uint4 nxt[NI];
    const bool more = base + step < p1;
    if (more) load(nxt, base + step);
    if (KL == KLOAD_STAGED) {
#pragma unroll
      for (int j = 0; j < NI; ++j)
        *reinterpret_cast<uint4*>(stage_rows + (j * RPI + lane / CPR) * PADB + (lane % CPR) * 16) = cur[j];
      lds_wave_sync();
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 a;
        if (KL == KLOAD_STAGED) a = *reinterpret_cast<const uint4*>(stage_rows + (16 * t + n) * PADB + (kg + 4 * s) * 16);
        else a = cur[t * KS + s];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bq[s], acc, 0, 0, 0);
      }
      const int pos = base + 16 * t + 4 * kg;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[i] * scale;
      if (MODE == MFMA_FULL && o.rmax) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kmax = pos + i < p1 ? max(kmax, score_key(v[i])) : kmax;
      }
      if (n < G) {
        if (MODE == MFMA_FULL) {
          float* Srow = o.S + row * L;
          if (vec_store && pos + 3 < p1) {
            *reinterpret_cast<float4*>(Srow + pos) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (pos + i < p1) Srow[pos + i] = v[i];
          }
        } else if (MODE == MFMA_SAMPLE) {
          float* Srow = o.S + row * o.nsamp + (p0 / chunk) * 64 - p0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (pos + i < p1) Srow[pos + i] = v[i];
        }
      }
    }
    if (KL == KLOAD_STAGED) __builtin_amdgcn_wave_barrier();  // reads of this round precede the next writes
    if (more) {
#pragma unroll
      for (int j = 0; j < NI; ++j) cur[j] = nxt[j];
    }
  }
  if (MODE == MFMA_FULL && o.rmax) {  // the four lanes of head n (rows kg = 0..3 of the wave) combine
    uint32_t e, od;
    rows_swap16(kmax, e, od);
    kmax = max(e, od);
    halves_swap32(kmax, e, od);
    kmax = max(e, od);
    if (lane < G) o.rmax[row * o.rmax_slots + blockIdx.x * 4 + wave] = kmax;
  }
}

// ---------------------------------------------------------------------------
// Candidate scan, persistent form (the hot loop of the fused exact step).
// PS_WPC workgroups per CU; workgroup i owns a contiguous, balanced range of
// 32-position tiles of the flattened (batch * KV head, position) space, and
// its waves take every fourth tile, so each wave streams K without gaps
// (next tile prefetched while the current one is scored). K goes through the
// wave's padded LDS rows as in KLOAD_STAGED. Kept means "ranks at or above
// T[row]" in the select order: key(s) >= key(T), which for fp32 is s >= T,
// plus everything when T is NaN (NaN scores never rank at or above a number).
// Kept (score, position) pairs are staged per head in wave-private LDS and
// handed to the rows' lists when a head's stage could overflow on the next
// tile, before the wave moves to another KV head, and at the end. A flush is
// split around the next tile's loads: lanes 0..G-1 reserve list space for
// all heads with one atomic instruction, the loads go out, then the staged
// pairs are copied, so waiting for the reservation never drains the wave's
// loads. Tile addresses and the (group, tile) cursor advance incrementally.
// ---------------------------------------------------------------------------
#ifndef TKA_PS_WPC
#define TKA_PS_WPC 2
#endif
#ifndef TKA_PS_STAGE_BYTES
#define TKA_PS_STAGE_BYTES 11776
#endif
constexpr int PS_WPC = TKA_PS_WPC;                  // workgroups per CU
// candidate stage per wave: G heads x S slots of 6 bytes (4-byte score bits and a 16-bit position
// offset from the stage's first tile), plus 64 spare slots that take the writes of pairs not kept
constexpr int PS_STAGE_BYTES = TKA_PS_STAGE_BYTES;
constexpr int PS_TILE_MAX = 32;                     // most pairs one head can keep from one tile
#ifndef TKA_PS_GUARD
#define TKA_PS_GUARD 4
#endif
constexpr int PS_GUARD = TKA_PS_GUARD;  // free slots per head below which the next tile is preceded by a flush

template <int D, bool SH>
__global__ __launch_bounds__(256) void score_cand_persistent_kernel(const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ K, int Hq, int Hkv,
                                                                    int G, int M, int L, int64_t sb, int64_t sh,
                                                                    int64_t sl, float scale, int64_t ntiles, int tpg,
                                                                    int S, MfmaOut o) {
  constexpr int KS = D / 32;
  constexpr int P = 32;
  constexpr int RB = D * 2, PADB = RB + 16, CPR = RB / 16, RPI = 1024 / RB, NI = P / RPI;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: the tile cursor lives in SGPRs
  const int n = lane & 15, kg = lane >> 4;
  // M queries per sequence (M <= 4): wave w scores query tq = w % M on tile lane w / M of TL = 4 / M;
  // the M waves of a tile lane read the same tiles (SH: cached loads, so the repeats hit the caches)
  const int TL = 4 / M;
  if (wave >= M * TL) return;
  const int tq = wave % M;
  const int lim = L - M + tq + 1;  // positions query tq may see
  extern __shared__ uint4 smem_raw[];
  uint8_t* rows = reinterpret_cast<uint8_t*>(smem_raw) + (size_t)wave * P * PADB;
  // S (score bits, position) slots per head, then one spare slot per lane that takes the writes
  // of pairs not kept (a slot per lane: one shared slot would make every such write a conflict).
  // A slot is 6 bytes: the score bits, and the position as a 16-bit offset from pbase, the first
  // position of the stage's first tile (so a stage holds a third more pairs than at 8 bytes)
  const int NS = G * S + 64;
  uint32_t* sbits = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(smem_raw) + (size_t)4 * P * PADB +
                                                (size_t)wave * NS * 6);
  uint16_t* soff = reinterpret_cast<uint16_t*>(sbits + NS);
  int pbase = 0;

  const int64_t per = ntiles / gridDim.x, extra = ntiles % gridDim.x;
  const int64_t r0 = blockIdx.x * per + min((int64_t)blockIdx.x, extra);
  const int64_t r1 = r0 + per + ((int64_t)blockIdx.x < extra ? 1 : 0);

  int grp = -1;           // KV group (b * Hkv + g) whose fragments are loaded
  bf16x8_t bq[KS];
  float Tf = 0.f;         // head n's threshold
  bool tnan = false;
  uint32_t scnt = 0;      // staged pairs of head n (lanes with n < G)
  const bool hl = n < G;  // this lane holds a head

  // reserve list space for every head's staged pairs: lane h < G holds head h's count
  auto reserve = [&]() -> uint32_t {
    const int b = grp / Hkv, g = grp % Hkv;
    uint32_t base = 0;
    if (lane < G && scnt != 0) base = atomicAdd(&o.cnt[((int64_t)b * M + tq) * Hq + g * G + lane], scnt);
    return base;
  };
  // copy the staged pairs to the reserved slots (counts and bases broadcast from lane h)
  auto copy_out = [&](uint32_t base) {
    const int b = grp / Hkv, g = grp % Hkv;
    const int64_t rg = ((int64_t)b * M + tq) * Hq + g * G;
    for (int h = 0; h < G; ++h) {
      const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)scnt, h);
      if (c == 0) continue;
      const uint32_t bh = (uint32_t)__builtin_amdgcn_readlane((int)base, h);
      const int64_t r = rg + h;
      if (o.cpair) {  // one 8-byte (bits, position) store per pair
        for (uint32_t e = lane; e < c; e += 64)
          if (bh + e < (uint32_t)o.capg) {  // streaming stores: the lists are read once, by another kernel
            u32x2_t x = {sbits[h * S + e], (uint32_t)pbase + soff[h * S + e]};
            __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(o.cpair + r * o.capg + bh + e));
          }
      } else {
        for (uint32_t e = lane; e < c; e += 64)
          if (bh + e < (uint32_t)o.capg) {
            __builtin_nontemporal_store(sbits[h * S + e], o.cbits + r * o.capg + bh + e);
            __builtin_nontemporal_store(pbase + (int32_t)soff[h * S + e], o.cpos + r * o.capg + bh + e);
          }
      }
    }
    scnt = 0;
  };
  // K rows of tile `tin` of group `g`: whole tiles step by a fixed stride, the last
  // (partial) tile of a group clamps its rows to L-1
  const int64_t jstep = (int64_t)RPI * sl;
  int lg = -1;
  const uint16_t* lK = K;
  auto load = [&](uint4 (&a)[NI], int g, int tin) {
    if (g != lg) {
      lg = g;
      lK = K + (int64_t)(g / Hkv) * sb + (int64_t)(g % Hkv) * sh + (lane % CPR) * 8;
    }
    const int at = tin * P;
    if (at + P <= L) {
      const uint16_t* p = lK + (int64_t)(at + lane / CPR) * sl;
#pragma unroll
      for (int j = 0; j < NI; ++j) a[j] = SH ? ld16(p + j * jstep) : ld16_stream(p + j * jstep);
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int pos = min(at + j * RPI + lane / CPR, L - 1);
        a[j] = SH ? ld16(lK + (int64_t)pos * sl) : ld16_stream(lK + (int64_t)pos * sl);
      }
    }
  };

  // tile t = cg * tpg + ct; each tile lane takes every TL-th tile of [r0, r1)
  int64_t t = r0 + wave / M;
  int cg = 0, ct = 0;
  uint4 cur[NI];
  if (t < r1) {
    cg = (int)(t / tpg);
    ct = (int)(t % tpg);
    load(cur, cg, ct);
  }
  pbase = ct * P;
  bool pend = false;  // wave-uniform: flush the stage before this tile's pairs are staged
  for (; t < r1; t += TL) {
    int ng = cg, nt = ct + TL;  // the wave's next tile
    while (nt >= tpg) {
      nt -= tpg;
      ++ng;
    }
    const uint32_t base = pend ? reserve() : 0u;
    uint4 nxt[NI];
    const bool more = t + TL < r1;
    if (more) load(nxt, ng, nt);
    if (pend) {
      copy_out(base);
      pend = false;
      pbase = ct * P;  // the stage is empty: offsets count from this tile
    }
    if (cg != grp) {  // new KV group (its stage is empty): load the fragments and thresholds
      grp = cg;
      const int b = grp / Hkv, g = grp % Hkv;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hl) v = ld16(q + (((int64_t)b * M + tq) * Hq + g * G + n) * D + 32 * s + 8 * kg);
        bq[s] = __builtin_bit_cast(bf16x8_t, v);
      }
      const float tv = hl ? o.T[((int64_t)b * M + tq) * Hq + g * G + n] : 0.f;
      Tf = tv;
      tnan = tv != tv;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j)
      *reinterpret_cast<uint4*>(rows + (j * RPI + lane / CPR) * PADB + (lane % CPR) * 16) = cur[j];
    lds_wave_sync();
    const int pos0 = ct * P;
    const bool whole = pos0 + P <= lim;
    bool f[2][4];
    float v[2][4];
    uint32_t c = 0;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(rows + (16 * tt + n) * PADB + (kg + 4 * s) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bq[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[tt][i] = acc[i] * scale;
        f[tt][i] = hl & (tnan | (v[tt][i] >= Tf));
      }
    }
    if (!whole) {  // the last tile: rows past the query's limit (loaded as row L-1) are never kept
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) f[tt][i] = f[tt][i] & (pos0 + 16 * tt + 4 * kg + i < lim);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) c += f[tt][i] ? 1u : 0u;
    __builtin_amdgcn_wave_barrier();  // operand reads of this tile precede the next tile's writes
    // per head: total over the four lanes holding it (rows kg = 0..3 of the wave), and this lane's
    // offset among them (kg order): row swaps give each row pair's counts, then each half's
    uint32_t c0, c1, p0, p1;
    rows_swap16(c, c0, c1);
    const uint32_t pair = c0 + c1;
    halves_swap32(pair, p0, p1);
    const uint32_t tot = p0 + p1;
    const uint32_t pre = ((kg & 1) ? c0 : 0u) + ((kg & 2) ? p0 : 0u);
    // a head that cannot take this tile's pairs: flush now (the deferred flush below reserves only
    // PS_GUARD slots, so this exact test catches the rarer tiles that keep more)
    if (PS_GUARD < PS_TILE_MAX && ballot(lane < 16 && hl && scnt + tot > (uint32_t)S) != 0) {
      copy_out(reserve());
      pbase = ct * P;
    }
    {  // scnt + tot <= S: the stage was flushed when it could not take this tile. No branches:
       // a pair not kept (and every pair of a lane without a head) goes to the lane's spare slot
      const uint32_t hs = (uint32_t)(n * S), sp = (uint32_t)(G * S + lane);
      uint32_t slot = scnt + pre;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t e = f[tt][i] ? hs + slot : sp;
          sbits[e] = __float_as_uint(v[tt][i]);
          soff[e] = (uint16_t)(pos0 + 16 * tt + 4 * kg + i - pbase);
          slot += f[tt][i] ? 1u : 0u;
        }
      if (hl) scnt += tot;
    }
    // flush before the next tile if a head is nearly full (a fuller tile is caught by the exact test
    // before staging), it starts another group, or its positions would not fit 16-bit offsets from
    // the stage's first tile
    pend = more && (ng != cg || nt * P + (P - 1) - pbase > 65535 ||
                    ballot(lane < 16 && hl && scnt > (uint32_t)(S - PS_GUARD)) != 0);
    if (more) {
#pragma unroll
      for (int j = 0; j < NI; ++j) cur[j] = nxt[j];
    }
    cg = ng;
    ct = nt;
  }
  if (grp >= 0) copy_out(reserve());
}

// ---------------------------------------------------------------------------
// Candidate scan for several queries per sequence with R = M * G <= 16 * NBLK
// (query, head) rows per KV group, persistent like the one-query scan: each
// wave streams its own tiles (every fourth of the workgroup's range) through
// its padded LDS rows, with no workgroup barrier, and scores all R rows of the
// group on each tile: the rows fill the 16 columns of NBLK MFMA blocks (column
// n of block cb is row cb * 16 + n: query (cb * 16 + n) / G, head
// (cb * 16 + n) % G), so K is read once for every query and no column is
// padding when R is a multiple of 16. Each lane keeps its rows' fragments,
// thresholds and causal limits (L - M + t + 1); staging, flushes and the list
// reservation work per row as in the one-query scan, over R rows.
// ---------------------------------------------------------------------------
template <int D, int NBLK>
__global__ __launch_bounds__(256) void score_cand_rows_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ K, int Hq, int Hkv,
                                                              int G, int M, int L, int64_t sb, int64_t sh,
                                                              int64_t sl, float scale, int64_t ntiles, int tpg,
                                                              int S, MfmaOut o) {
  constexpr int KS = D / 32;
  constexpr int P = 32;
  constexpr int RB = D * 2, PADB = RB + 16, CPR = RB / 16, RPI = 1024 / RB, NI = P / RPI;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int R = M * G;
  bool hl[NBLK];
  int tq[NBLK], hh[NBLK], lim[NBLK];
#pragma unroll
  for (int cb = 0; cb < NBLK; ++cb) {
    const int rr = cb * 16 + n;
    hl[cb] = rr < R;
    tq[cb] = hl[cb] ? rr / G : 0;
    hh[cb] = hl[cb] ? rr % G : 0;
    lim[cb] = L - M + tq[cb] + 1;  // positions this row's query may see
  }
  const int lim_all = L - M + 1;  // ... that every query may see
  extern __shared__ uint4 smem_raw[];
  uint8_t* rows = reinterpret_cast<uint8_t*>(smem_raw) + (size_t)wave * P * PADB;
  // S slots per row (R rows), then one spare slot per lane; 6-byte slots as in the one-query scan
  const int NS = R * S + 64;
  uint32_t* sbits = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(smem_raw) + (size_t)4 * P * PADB +
                                                (size_t)wave * NS * 6);
  uint16_t* soff = reinterpret_cast<uint16_t*>(sbits + NS);
  int pbase = 0;

  const int64_t per = ntiles / gridDim.x, extra = ntiles % gridDim.x;
  const int64_t r0 = blockIdx.x * per + min((int64_t)blockIdx.x, extra);
  const int64_t r1 = r0 + per + ((int64_t)blockIdx.x < extra ? 1 : 0);

  int grp = -1;
  bf16x8_t bq[NBLK][KS];
  float Tf[NBLK];
  bool tnan[NBLK];
  uint32_t scnt[NBLK];  // staged pairs of row cb * 16 + n (every lane of column n holds it)
#pragma unroll
  for (int cb = 0; cb < NBLK; ++cb) {
    Tf[cb] = 0.f;
    tnan[cb] = false;
    scnt[cb] = 0;
  }
  auto row_of = [&](int cb) -> int64_t {
    const int b = grp / Hkv, g = grp % Hkv;
    return ((int64_t)b * M + tq[cb]) * Hq + g * G + hh[cb];
  };
  // list space for every row's staged pairs: lane n < 16 reserves for row cb * 16 + n
  auto reserve = [&](uint32_t (&base)[NBLK]) {
#pragma unroll
    for (int cb = 0; cb < NBLK; ++cb) {
      base[cb] = 0;
      if (lane < 16 && hl[cb] && scnt[cb] != 0) base[cb] = atomicAdd(&o.cnt[row_of(cb)], scnt[cb]);
    }
  };
  auto copy_out = [&](const uint32_t (&base)[NBLK]) {
    const int b = grp / Hkv, g = grp % Hkv;
#pragma unroll
    for (int cb = 0; cb < NBLK; ++cb) {
      for (int h = 0; h < 16; ++h) {
        const int rr = cb * 16 + h;
        const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)scnt[cb], h);
        if (rr >= R || c == 0) continue;  // wave-uniform
        const uint32_t bh = (uint32_t)__builtin_amdgcn_readlane((int)base[cb], h);
        const int64_t r = ((int64_t)b * M + rr / G) * Hq + g * G + rr % G;
        if (o.cpair) {
          for (uint32_t e = lane; e < c; e += 64)
            if (bh + e < (uint32_t)o.capg) {
              u32x2_t x = {sbits[rr * S + e], (uint32_t)pbase + soff[rr * S + e]};
              __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(o.cpair + r * o.capg + bh + e));
            }
        } else {
          for (uint32_t e = lane; e < c; e += 64)
            if (bh + e < (uint32_t)o.capg) {
              __builtin_nontemporal_store(sbits[rr * S + e], o.cbits + r * o.capg + bh + e);
              __builtin_nontemporal_store(pbase + (int32_t)soff[rr * S + e], o.cpos + r * o.capg + bh + e);
            }
        }
      }
      scnt[cb] = 0;
    }
  };
  auto flush = [&]() {
    uint32_t base[NBLK];
    reserve(base);
    copy_out(base);
  };
  const int64_t jstep = (int64_t)RPI * sl;
  int lg = -1;
  const uint16_t* lK = K;
  auto load = [&](uint4 (&a)[NI], int g, int tin) {
    if (g != lg) {
      lg = g;
      lK = K + (int64_t)(g / Hkv) * sb + (int64_t)(g % Hkv) * sh + (lane % CPR) * 8;
    }
    const int at = tin * P;
    if (at + P <= L) {
      const uint16_t* p = lK + (int64_t)(at + lane / CPR) * sl;
#pragma unroll
      for (int j = 0; j < NI; ++j) a[j] = ld16_stream(p + j * jstep);
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int pos = min(at + j * RPI + lane / CPR, L - 1);
        a[j] = ld16_stream(lK + (int64_t)pos * sl);
      }
    }
  };

  int64_t t = r0 + wave;  // this wave takes every fourth tile of [r0, r1)
  int cg = 0, ct = 0;
  uint4 cur[NI];
  if (t < r1) {
    cg = (int)(t / tpg);
    ct = (int)(t % tpg);
    load(cur, cg, ct);
  }
  pbase = ct * P;
  bool pend = false;  // wave-uniform: flush the stage before this tile's pairs are staged
  for (; t < r1; t += 4) {
    int ng = cg, nt = ct + 4;
    while (nt >= tpg) {
      nt -= tpg;
      ++ng;
    }
    uint32_t base[NBLK];
    if (pend) reserve(base);
    uint4 nxt[NI];
    const bool more = t + 4 < r1;
    if (more) load(nxt, ng, nt);
    if (pend) {
      copy_out(base);
      pend = false;
      pbase = ct * P;
    }
    if (cg != grp) {  // new KV group (its stage is empty): the rows' fragments and thresholds
      grp = cg;
#pragma unroll
      for (int cb = 0; cb < NBLK; ++cb) {
        const int64_t qr = row_of(cb);
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (hl[cb]) v = ld16(q + qr * D + 32 * s2 + 8 * kg);
          bq[cb][s2] = __builtin_bit_cast(bf16x8_t, v);
        }
        const float tv = hl[cb] ? o.T[qr] : 0.f;
        Tf[cb] = tv;
        tnan[cb] = tv != tv;
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j)
      *reinterpret_cast<uint4*>(rows + (j * RPI + lane / CPR) * PADB + (lane % CPR) * 16) = cur[j];
    lds_wave_sync();
    const int pos0 = ct * P;
    const bool whole = pos0 + P <= lim_all;
    bool f[NBLK][2][4];
    float v[NBLK][2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4_t acc[NBLK];
#pragma unroll
      for (int cb = 0; cb < NBLK; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) {
        const uint4 a = *reinterpret_cast<const uint4*>(rows + (16 * tt + n) * PADB + (kg + 4 * s2) * 16);
#pragma unroll
        for (int cb = 0; cb < NBLK; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bq[cb][s2], acc[cb], 0,
                                                            0, 0);
      }
#pragma unroll
      for (int cb = 0; cb < NBLK; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[cb][tt][i] = acc[cb][i] * scale;
          f[cb][tt][i] = hl[cb] & (tnan[cb] | (v[cb][tt][i] >= Tf[cb]));
        }
    }
    if (!whole) {  // the last tiles: positions past a row's query limit (or past L) are never kept
#pragma unroll
      for (int cb = 0; cb < NBLK; ++cb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) f[cb][tt][i] = f[cb][tt][i] & (pos0 + 16 * tt + 4 * kg + i < lim[cb]);
    }
    __builtin_amdgcn_wave_barrier();  // operand reads of this tile precede the next tile's writes
    uint32_t tot[NBLK], pre[NBLK];
    bool over = false;
#pragma unroll
    for (int cb = 0; cb < NBLK; ++cb) {
      uint32_t c = 0;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) c += f[cb][tt][i] ? 1u : 0u;
      uint32_t c0, c1, p0, p1;  // a row's total over its four lanes and this lane's offset (kg order)
      rows_swap16(c, c0, c1);
      const uint32_t pair = c0 + c1;
      halves_swap32(pair, p0, p1);
      tot[cb] = p0 + p1;
      pre[cb] = ((kg & 1) ? c0 : 0u) + ((kg & 2) ? p0 : 0u);
      over = over || (hl[cb] && scnt[cb] + tot[cb] > (uint32_t)S);
    }
    // a row that cannot take this tile's pairs: flush now
    if (ballot(lane < 16 && over) != 0) {
      flush();
      pbase = ct * P;
    }
    {  // no branches: a pair not kept goes to the lane's spare slot
      const uint32_t sp = (uint32_t)(R * S + lane);
#pragma unroll
      for (int cb = 0; cb < NBLK; ++cb) {
        const uint32_t hs = (uint32_t)((cb * 16 + n) * S);
        uint32_t slot = scnt[cb] + pre[cb];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t e = f[cb][tt][i] ? hs + slot : sp;
            sbits[e] = __float_as_uint(v[cb][tt][i]);
            soff[e] = (uint16_t)(pos0 + 16 * tt + 4 * kg + i - pbase);
            slot += f[cb][tt][i] ? 1u : 0u;
          }
        if (hl[cb]) scnt[cb] += tot[cb];
      }
    }
    bool near = false;
#pragma unroll
    for (int cb = 0; cb < NBLK; ++cb) near = near || (hl[cb] && scnt[cb] > (uint32_t)(S - PS_GUARD));
    pend = more && (ng != cg || nt * P + (P - 1) - pbase > 65535 || ballot(lane < 16 && near) != 0);
    if (more) {
#pragma unroll
      for (int j = 0; j < NI; ++j) cur[j] = nxt[j];
    }
    cg = ng;
    ct = nt;
  }
  if (grp >= 0) flush();
}

// ---------------------------------------------------------------------------
// Candidate scan for several queries per sequence (2 <= M <= 4) with more
// than 32 (query, head) rows per KV group, persistent.
// Workgroup i owns a contiguous range of 32-position tiles of the flattened
// (batch * KV head, position) space, as above, but its four waves take every
// tile together: the workgroup loads a tile once (each thread 16-byte chunks
// of it), four tiles ahead in a ring of four register buffers written out by
// hand, stores it to one of two LDS tile buffers, and after one barrier wave
// w < M scores query w's G heads on it (the MFMA, threshold test, staging
// and flushes of the one-query scan, with the query's causal limit).
// ---------------------------------------------------------------------------
#ifndef TKA_SHARED_SCAN
#define TKA_SHARED_SCAN 1
#endif
#ifndef TKA_ROWS_SCAN
#define TKA_ROWS_SCAN 1
#endif
#ifndef TKA_SS_GUARD
#define TKA_SS_GUARD 8
#endif
// free stage slots per row below which a flush is scheduled before the next tile (a tile that
// would overflow anyway is preceded by an immediate flush)
constexpr int SS_GUARD = TKA_SS_GUARD;
#ifndef TKA_SS_WPC
#define TKA_SS_WPC 2
#endif
constexpr int SS_WPC = TKA_SS_WPC;  // workgroups per CU

template <int D, int NTT>
__global__ __launch_bounds__(256) void score_cand_shared_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ K, int Hq, int Hkv,
                                                                int G, int M, int L, int64_t sb, int64_t sh,
                                                                int64_t sl, float scale, int ntiles, int tpg, int S,
                                                                MfmaOut o) {
  constexpr int KS = D / 32;
  constexpr int P = 32;
  constexpr int RB = D * 2, PADB = RB + 16, CPR = RB / 16;
  constexpr int NT = P * CPR / 256;  // 16-byte chunks a thread loads per tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kg = lane >> 4;
  // the R = M * G (query, head) rows of a KV group in blocks of 16 (lane column n: query t = row / G,
  // head row % G), so every MFMA column and epilogue lane works. NTT = 2: wave w scores block w on
  // both 16-position halves of a tile; NTT = 1 (at most two blocks): wave w scores block w / 2 on
  // half w % 2, so that four waves share the work
  const int R = M * G;
  const int cb = NTT == 1 ? wave >> 1 : wave, half = NTT == 1 ? wave & 1 : 0;
  const bool act = cb * 16 < R;
  const int rr = cb * 16 + n;  // this lane's row (column) of the group
  const bool hl = act && rr < R;
  const int tl = hl ? rr / G : 0, hh = hl ? rr % G : 0;
  const int lim = L - M + tl + 1;    // positions the lane's query may see
  const int lim_all = L - M + 1;     // ... that every query may see
  extern __shared__ uint4 smem_raw[];
  uint8_t* tiles = reinterpret_cast<uint8_t*>(smem_raw);  // two tile buffers of P rows
  // S slots per row, then one spare slot per lane (pairs not kept); stages of the scoring waves only
  uint2* stg = reinterpret_cast<uint2*>(tiles + 2 * P * PADB) + (size_t)(act ? wave : 0) * (16 * S + 64);
  uint2* const spare = stg + 16 * S + lane;

  const int per = ntiles / (int)gridDim.x, extra = ntiles % (int)gridDim.x;
  const int r0 = (int)blockIdx.x * per + min((int)blockIdx.x, extra);
  const int r1 = r0 + per + ((int)blockIdx.x < extra ? 1 : 0);
  if (r0 >= r1) return;  // workgroup-uniform

  int grp = -1;
  bf16x8_t bq[KS];
  float Tf = 0.f;
  bool tnan = false;
  uint32_t scnt = 0;
  // list of the lane's row in group grp: ((b * M + t) * Hq + g * G + head)
  auto row_of = [&](int t, int head) -> int64_t {
    const int b = grp / Hkv, g = grp % Hkv;
    return ((int64_t)b * M + t) * Hq + g * G + head;
  };
  auto reserve = [&]() -> uint32_t {
    uint32_t base = 0;
    if (lane < 16 && scnt != 0) base = atomicAdd(&o.cnt[row_of(tl, hh)], scnt);
    return base;
  };
  const bool packed = o.cpair != nullptr;  // kernel-uniform
  auto copy_out = [&](uint32_t base) {
    for (int h = 0; h < 16; ++h) {
      const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)scnt, h);
      if (c == 0) continue;  // (columns past R never count)
      const uint32_t bh = (uint32_t)__builtin_amdgcn_readlane((int)base, h);
      const int rc = cb * 16 + h;
      const int64_t r = row_of(rc / G, rc % G);
      for (uint32_t e = lane; e < c; e += 64)
        if (bh + e < (uint32_t)o.capg) {
          const uint2 y = stg[h * S + e];
          if (packed) {  // the fused step's packed lists
            u32x2_t x = {y.x, y.y};
            __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(o.cpair + r * o.capg + bh + e));
          } else {  // separate score-bit and position lists (the thresholded-scan entry)
            __builtin_nontemporal_store(y.x, o.cbits + r * o.capg + bh + e);
            __builtin_nontemporal_store((int32_t)y.y, o.cpos + r * o.capg + bh + e);
          }
        }
    }
    scnt = 0;
  };
  // loads of tile u into a (rows past L-1 re-read row L-1); past the range's last tile the
  // cursor stays on it, so every step issues the same number of loads
  // (tile cursors advance incrementally: a division per step costs dozens of scalar instructions)
  int ld = r0, lg = r0 / tpg, lt = r0 - lg * tpg;
  const uint16_t* lbase = K + (int64_t)(lg / Hkv) * sb + (int64_t)(lg % Hkv) * sh;
  auto load_next = [&](uint4 (&a)[NT]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = tid + 256 * j;
      const int pos = min(lt * P + c / CPR, L - 1);
      a[j] = ld16(lbase + (int64_t)pos * sl + (c % CPR) * 8);
    }
    if (ld + 1 < r1) {
      ++ld;
      if (++lt == tpg) {
        lt = 0;
        ++lg;
        lbase = K + (int64_t)(lg / Hkv) * sb + (int64_t)(lg % Hkv) * sh;
      }
    }
  };
  int u = r0;  // the tile being scored
  int cg = r0 / tpg, ct = r0 - cg * tpg;  // ... as (group, tile in group)
  bool pend = false;
  // one tile: its registers to LDS, the buffer refilled SS_DEPTH tiles ahead, a barrier, the scoring.
  // Steps past the range (rounding the loop up to whole rounds) only load and meet the barrier.
  auto step = [&](uint4 (&a)[NT]) {
    const bool live = u < r1;  // workgroup-uniform
    uint8_t* tb = tiles + (size_t)(u & 1) * P * PADB;
    if (live) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int c = tid + 256 * j;
        *reinterpret_cast<uint4*>(tb + (c / CPR) * PADB + (c % CPR) * 16) = a[j];
      }
    }
    load_next(a);
    __syncthreads();  // the tile is in LDS; every wave is done with the buffer written next step
    const bool more = u + 1 < r1;
    if (live && act) {
      if (pend) {
        copy_out(reserve());
        pend = false;
      }
      if (cg != grp) {  // new KV group (its stage is empty): the rows' fragments and thresholds
        grp = cg;
        const int64_t qr = row_of(tl, hh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          uint4 v = make_uint4(0, 0, 0, 0);
          if (hl) v = ld16(q + qr * D + 32 * s + 8 * kg);
          bq[s] = __builtin_bit_cast(bf16x8_t, v);
        }
        const float tv = hl ? o.T[qr] : 0.f;
        Tf = tv;
        tnan = tv != tv;
      }
      const int pos0 = ct * P;
      const bool whole = pos0 + P <= lim_all;  // wave-uniform
      bool f[NTT][4];
      float v[NTT][4];
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
        const int tt = NTT == 1 ? half : j;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const uint4 x = *reinterpret_cast<const uint4*>(tb + (16 * tt + n) * PADB + (kg + 4 * s) * 16);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), bq[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[j][i] = acc[i] * scale;
          f[j][i] = hl & (tnan | (v[j][i] >= Tf));
        }
      }
      if (!whole) {
#pragma unroll
        for (int j = 0; j < NTT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            f[j][i] = f[j][i] & (pos0 + 16 * (NTT == 1 ? half : j) + 4 * kg + i < lim);
      }
#pragma unroll
      for (int j = 0; j < NTT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) c += f[j][i] ? 1u : 0u;
      uint32_t c0, c1, p0, p1;  // row and half swaps, as in the one-query scan
      rows_swap16(c, c0, c1);
      const uint32_t pair = c0 + c1;
      halves_swap32(pair, p0, p1);
      const uint32_t tot = p0 + p1;
      const uint32_t pre = ((kg & 1) ? c0 : 0u) + ((kg & 2) ? p0 : 0u);
      // a row that cannot take this tile's pairs: flush now (the deferred flush below reserves
      // only SS_GUARD slots, so this exact test catches the rarer tiles that keep more)
      if (SS_GUARD < PS_TILE_MAX && ballot(lane < 16 && hl && scnt + tot > (uint32_t)S) != 0) copy_out(reserve());
      {
        uint2* hs = stg + n * S;
        uint32_t slot = scnt + pre;
#pragma unroll
        for (int j = 0; j < NTT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            *(f[j][i] ? hs + slot : spare) =
                make_uint2(__float_as_uint(v[j][i]), (uint32_t)(pos0 + 16 * (NTT == 1 ? half : j) + 4 * kg + i));
            slot += f[j][i] ? 1u : 0u;
          }
        if (hl) scnt += tot;
      }
      pend = more && (ct + 1 == tpg || ballot(lane < 16 && hl && scnt > (uint32_t)(S - SS_GUARD)) != 0);
    }
    ++u;
    if (++ct == tpg) {
      ct = 0;
      ++cg;
    }
  };
  // whole rounds of four steps, one exit at the bottom: a loop left from the middle of a round
  // gets one merged exit test that can branch back to the top, and on that path the compiler
  // must assume the buffer just refilled is needed at once, draining every load in flight
  // (the scheduling barriers keep the four buffers' loads in this order: if the scheduler issued
  // a0's last, the one wait the compiler places for a0 would have to drain everything)
  uint4 a0[NT], a1[NT], a2[NT], a3[NT];
  load_next(a0);
  __builtin_amdgcn_sched_barrier(0);
  load_next(a1);
  __builtin_amdgcn_sched_barrier(0);
  load_next(a2);
  __builtin_amdgcn_sched_barrier(0);
  load_next(a3);
  __builtin_amdgcn_sched_barrier(0);
  const int rounds = (r1 - r0 + 3) / 4;
  for (int rd = 0; rd < rounds; ++rd) {
    step(a0);
    step(a1);
    step(a2);
    step(a3);
  }
  if (act && grp >= 0) copy_out(reserve());
}

// ---------------------------------------------------------------------------
// Several causal queries per sequence ("Evolution of Sparse Attention in
// Long-Context LLMs", section 6: current length x K instead of current length
// x full history): the M queries of sequence b sit at positions L-M .. L-1
// and query t sees keys 0 .. L-M+t. The R = M*G (query, head) rows of a KV
// group share every key row, so the score is a real contraction: a K tile is
// staged once through LDS (as in KLOAD_STAGED) and each of its 16x32 operand
// fragments feeds RT row tiles of 16 rows (v_mfma_f32_16x16x32_bf16; lane l of
// row tile rt holds row rt*16 + l%16 = t*G + hh). Scores go to row
// (b*M + t)*Hq + g*G + hh of [B*M*Hq, L]; positions past the query's own are
// NaN (they rank below every number). Grid (chunks, B*Hkv), 256 threads.
// ---------------------------------------------------------------------------
enum { MQ_FULL = 0, MQ_SAMPLE = 1 };
template <int D, int RT, int MODE>
__global__ __launch_bounds__(256) void score_mq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ K,
                                                       int Hq, int Hkv, int G, int M, int L, int64_t sb, int64_t sh,
                                                       int64_t sl, float scale, int chunk, float* __restrict__ S,
                                                       int nsamp) {
  constexpr int KS = D / 32;
  constexpr int P = 32;
  constexpr int RB = D * 2, PADB = RB + 16, CPR = RB / 16, RPI = 1024 / RB, NI = P / RPI;
  const int task = blockIdx.y;
  const int b = task / Hkv, g = task % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int R = M * G;
  extern __shared__ uint4 smem_raw[];
  uint8_t* rows = reinterpret_cast<uint8_t*>(smem_raw) + (size_t)wave * P * PADB;

  bf16x8_t bq[RT][KS];
  int64_t srow[RT];
  int last[RT];  // the last position row rt of this lane may see
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + n;
    const bool ok = rr < R;
    const int t = ok ? rr / G : 0, hh = ok ? rr % G : 0;
    const int64_t qr = ((int64_t)b * M + t) * Hq + g * G + hh;
    srow[rt] = ok ? qr : -1;
    last[rt] = L - M + t;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = ld16(q + qr * D + 32 * s + 8 * kg);
      bq[rt][s] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const uint16_t* Kb = K + (int64_t)b * sb + (int64_t)g * sh;
  // sample mode: the first 64 positions of sample chunk blockIdx.x, to samples blockIdx.x*64 + ...
  const int p0 = blockIdx.x * chunk, p1 = min(p0 + (MODE == MQ_SAMPLE ? 64 : chunk), L);
  const bool vec_store = MODE != MQ_SAMPLE && (L & 3) == 0;
  auto load = [&](uint4 (&a)[NI], int at) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int pos = min(at + j * RPI + lane / CPR, L - 1);
      a[j] = ld16_stream(Kb + (int64_t)pos * sl + (lane % CPR) * 8);
    }
  };
  int base = p0 + wave * P;
  uint4 cur[NI];
  if (base < p1) load(cur, base);
  for (; base < p1; base += 4 * P) {
    uint4 nxt[NI];
    const bool more = base + 4 * P < p1;
    if (more) load(nxt, base + 4 * P);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      *reinterpret_cast<uint4*>(rows + (j * RPI + lane / CPR) * PADB + (lane % CPR) * 16) = cur[j];
    lds_wave_sync();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      uint4 a[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        a[s] = *reinterpret_cast<const uint4*>(rows + (16 * tt + n) * PADB + (kg + 4 * s) * 16);
      const int pos = base + 16 * tt + 4 * kg;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]), bq[rt][s], acc, 0, 0, 0);
        if (srow[rt] >= 0) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = pos + i <= last[rt] ? acc[i] * scale : __int_as_float(0x7fc00000);
          float* Srow = MODE == MQ_SAMPLE ? S + srow[rt] * nsamp + (int64_t)blockIdx.x * 64 - p0 : S + srow[rt] * L;
          if (vec_store && pos + 3 < p1) {
            *reinterpret_cast<float4*>(Srow + pos) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (pos + i < p1) Srow[pos + i] = v[i];
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();  // reads of this round precede the next writes
    if (more) {
#pragma unroll
      for (int j = 0; j < NI; ++j) cur[j] = nxt[j];
    }
  }
}

__global__ void mq_counts_kernel(int32_t* __restrict__ krow, int64_t rows, int M, int Hq, int L, int k) {
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)((r / Hq) % M);
    krow[r] = min(k, L - M + t + 1);
  }
}

// ---------------------------------------------------------------------------
// Block-mean scores s[b,h,j] = <q[b,h], mean[b,g,j]> ("Sparse Attention
// Landscape", "Block Sparse Attention": the block score from the mean-pooled
// keys), fp32 means, the query bf16 or fp32. A row of D floats is read by a
// group of LPR lanes (8, or 16 for more than 4 heads), lane c taking the
// 16-byte pieces c, c + LPR, ... (a load instruction covers 16·LPR contiguous
// bytes of each of 64/LPR rows); each lane keeps the matching slices of the NH
// query heads, and the partial dots are summed over the row's lanes (DPP). A
// wave takes RND consecutive rounds of rows with all their loads issued before
// the first use.
// Grid (chunks, B*Hkv*htiles), 256 threads.
// ---------------------------------------------------------------------------
#ifndef TKA_BLK_LOADS
#define TKA_BLK_LOADS 8
#endif
template <int D, int NH>
struct BlockScoreShape {
  // lanes per row: 8, or 16 for more than 4 heads, so that the query slices a lane keeps (NH x its
  // pieces) stay at 64 registers
  static constexpr int LPR = NH > 4 ? 16 : 8;
  static constexpr int RPW = 64 / LPR;                     // rows per load instruction (per wave)
  static constexpr int NL = D / (4 * LPR) > 0 ? D / (4 * LPR) : 1;  // 16-byte pieces per lane
  static constexpr int LD = TKA_BLK_LOADS;                 // 16-byte loads in flight per lane
  static constexpr int RND = LD / NL > 0 ? LD / NL : 1;    // rounds of RPW rows in flight per wave
  static constexpr int ROWS = 4 * RPW * RND;               // rows per workgroup pass
};

template <int D, int NH>
__global__ __launch_bounds__(256) void score_block_kernel(const void* __restrict__ qv, const float* __restrict__ means,
                                                          float* __restrict__ S, int Hq, int Hkv, int G, int nrows,
                                                          int64_t sb, int64_t sh, int64_t sl, float scale, int chunk,
                                                          int htiles, int q_bf16) {
  using SH = BlockScoreShape<D, NH>;
  constexpr int NL = SH::NL, RND = SH::RND;
  const int task = blockIdx.y;
  const int ht = task % htiles, bg = task / htiles;
  const int b = bg / Hkv, g = bg % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % SH::LPR, grp = lane / SH::LPR;
  const int h0 = g * G + ht * NH;
  const int nh = min(NH, g * G + G - h0);
  float qf[NH][NL][4];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int64_t at = (int64_t)(b * Hq + h0 + h) * D + 4 * (sub + SH::LPR * j);
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (h < nh) {
        if (q_bf16) {
          const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(qv) + at);
          v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x); v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
        } else {
          const uint4 x = ld16(reinterpret_cast<const float*>(qv) + at);
          v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y);
          v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[h][j][e] = v[e];
    }
  const float* kb = means + (int64_t)b * sb + (int64_t)g * sh;
  const int p0 = blockIdx.x * chunk, p1 = min(p0 + chunk, nrows);
  for (int base = p0 + wave * SH::RPW * RND; base < p1; base += SH::ROWS) {
    uint4 raw[RND][NL];
#pragma unroll
    for (int r = 0; r < RND; ++r) {
      const int row = base + SH::RPW * r + grp;
#pragma unroll
      for (int j = 0; j < NL; ++j)
        raw[r][j] = row < p1 ? ld16_stream(kb + (int64_t)row * sl + 4 * (sub + SH::LPR * j)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < RND; ++r) {
      float part[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          x = fmaf(qf[h][j][0], __uint_as_float(raw[r][j].x), x);
          x = fmaf(qf[h][j][1], __uint_as_float(raw[r][j].y), x);
          x = fmaf(qf[h][j][2], __uint_as_float(raw[r][j].z), x);
          x = fmaf(qf[h][j][3], __uint_as_float(raw[r][j].w), x);
        }
        part[h] = x;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) part[h] = group_sum<SH::LPR>(part[h]);
      const int row = base + SH::RPW * r + grp;
      if (row < p1) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
          if (h == sub && h < nh) S[(int64_t)(b * Hq + h0 + h) * nrows + row] = part[h] * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wave dot-reduction scores for fp32 or bf16 rows, NH query heads per task.
// A row of D elements is 16*LPR bytes: LPR lanes load 16 B each, RPW = 64/LPR
// rows per wave load. Each lane keeps its 16-byte slice of q for every head,
// the partial dots are reduced across the LPR lanes with xor shuffles.
// Used for G = 1 heads, fp32 caches and the fp32 block-mean cache (whose
// query stays bf16: q_bf16 gives the query's dtype, BF16 the rows').
// Grid (chunks, B*Hkv*htiles), 256 threads.
// ---------------------------------------------------------------------------
template <bool BF16, int D, int NH>
__global__ __launch_bounds__(256) void score_vec_kernel(const void* __restrict__ qv, const void* __restrict__ Kv,
                                                        float* __restrict__ S, int Hq, int Hkv, int G, int nrows,
                                                        int64_t sb, int64_t sh, int64_t sl, float scale, int chunk,
                                                        int htiles, int q_bf16) {
  using U = Unpack<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = U::N;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int UNR = 4;
  const int task = blockIdx.y;
  const int ht = task % htiles;
  const int bg = task / htiles;
  const int b = bg / Hkv, g = bg % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, grp = lane / LPR;
  const int h0 = g * G + ht * NH;
  const int nh = min(NH, g * G + G - h0);

  float qf[NH][EPL];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int64_t q0 = (int64_t)(b * Hq + h0 + h) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = 0.f;
      if (h < nh)
        x = q_bf16 ? bf16_lo(reinterpret_cast<const uint16_t*>(qv)[q0 + e])
                   : reinterpret_cast<const float*>(qv)[q0 + e];
      qf[h][e] = x;
    }
  }
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(Kv) + ((int64_t)b * sb + (int64_t)g * sh) * ES;
  const int p0 = blockIdx.x * chunk;
  const int p1 = min(p0 + chunk, nrows);
  for (int base = p0 + wave * RPW * UNR; base < p1; base += 4 * RPW * UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int pos = min(base + u * RPW + grp, nrows - 1);
      raw[u] = ld16_stream(Kb + ((int64_t)pos * sl + sub * EPL) * ES);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[EPL];
      U::run(raw[u], kf);
      float part[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qf[h][e], kf[e], a);
        part[h] = a;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) part[h] = group_sum<LPR>(part[h]);
      const int pos = base + u * RPW + grp;
      if (pos < p1) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
          if (h % LPR == sub && h < nh) S[((int64_t)(b * Hq + h0 + h)) * nrows + pos] = part[h] * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Lightning-indexer scores, E4M3FN inputs, fp32 out (the MFMA core and its
// operand layout: indexer_core.h). Grid (chunks, B), 256 threads; each wave
// scores 32 * UNR positions per round.
// ---------------------------------------------------------------------------
template <int DI, int NT>
__global__ __launch_bounds__(256) void score_indexer_kernel(const uint8_t* __restrict__ qI,
                                                            const uint8_t* __restrict__ kI,
                                                            const float* __restrict__ w, float* __restrict__ S,
                                                            int HI, int L, int Lc, int chunk) {
  constexpr int UNR = 4;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, half = lane >> 5;
  IndexerQuery<DI, NT> Q;
  indexer_load_query<DI, NT>(Q, qI, w, b, HI, lane);
  const uint8_t* kb = kI + (int64_t)b * Lc * DI;
  float* Sb = S + (int64_t)b * L;
  const int p0 = blockIdx.x * chunk;
  const int p1 = min(p0 + chunk, L);
  for (int base = p0 + wave * 32 * UNR; base < p1; base += 4 * 32 * UNR) {
    float tot[UNR];
    indexer_round<DI, NT, UNR>(Q, kb, base, L, lane, tot);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int pos = base + 32 * u + j;
      if (half == 0 && pos < p1) Sb[pos] = tot[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Block means, fp32 out [B,Hkv,m,D]: one wave per block, lanes split a row
// into 16-byte slices, RPW rows per load; partial sums are combined across
// lane groups with xor shuffles. Grid (ceil(m/4), B*Hkv), 256 threads.
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) void block_mean_kernel(const void* __restrict__ Kv, float* __restrict__ means,
                                                         int Hkv, int L, int bsz, int m, int64_t sb, int64_t sh,
                                                         int64_t sl, int j0, int j1) {
  using U = Unpack<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = U::N;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = 64 / LPR;
  const int task = blockIdx.y;
  const int b = task / Hkv, g = task % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, grp = lane / LPR;
  const int j = j0 + blockIdx.x * 4 + wave;  // blocks [j0, j1) of the m
  if (j >= j1) return;
  const int i0 = j * bsz, i1 = min(i0 + bsz, L);
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(Kv) + ((int64_t)b * sb + (int64_t)g * sh) * ES;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int i = i0 + grp; i < i1; i += RPW) {
    float kf[EPL];
    U::run(ld16(Kb + ((int64_t)i * sl + sub * EPL) * ES), kf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += kf[e];
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = cross_sum<LPR>(acc[e]);
  if (grp == 0) {
    const float inv = 1.0f / (float)(i1 - i0);
    float* dst = means + (((int64_t)b * Hkv + g) * m + j) * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                                                         acc[e + 3] * inv);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int pick_chunk(int64_t rows_per_task, int64_t tasks, int granule, int lo, int hi) {
  // Enough workgroups to fill 256 CUs several times over, each streaming a
  // contiguous run of rows.
  int64_t c = hi;
  while (c > lo && tasks * ((rows_per_task + c - 1) / c) < 2048) c >>= 1;
  c = (c / granule) * granule;
  return (int)(c < granule ? granule : c);
}

template <int D, int MODE>
static void launch_mfma_mode(const ScoreArgs& a, int chunk, unsigned gx, const MfmaOut& o, hipStream_t st) {
  constexpr int KL = TKA_SCAN_KLOAD;
  const size_t lds = KL == KLOAD_STAGED ? (size_t)4 * 32 * (D * 2 + 16) : 0;
  dim3 grid(gx, a.B * a.Hkv);
  ensure_dynamic_lds((const void*)score_exact_mfma_kernel<D, MODE, KL>, lds);
  hipLaunchKernelGGL((score_exact_mfma_kernel<D, MODE, KL>), grid, dim3(256), lds, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, a.nrows, a.sb, a.sh, a.sl, a.scale, chunk, o);
}

template <int MODE>
static void launch_mfma(const ScoreArgs& a, int chunk, unsigned gx, const MfmaOut& o, hipStream_t st) {
  switch (a.d) {
    case 64: launch_mfma_mode<64, MODE>(a, chunk, gx, o, st); break;
    case 128: launch_mfma_mode<128, MODE>(a, chunk, gx, o, st); break;
    default: launch_mfma_mode<256, MODE>(a, chunk, gx, o, st); break;
  }
}

int mfma_scan_chunk(const ScoreArgs& a) { return pick_chunk(a.nrows, (int64_t)a.B * a.Hkv, 256, 256, 4096); }

template <int MODE>
static void launch_mq_mode(const ScoreArgs& a, int chunk, float* out, int nsamp, hipStream_t st);

void launch_score_mfma_sample(const ScoreArgs& a, int sample_chunk, int nsamp, float* samp, hipStream_t st) {
  if (a.M > 1) {
    launch_mq_mode<MQ_SAMPLE>(a, sample_chunk, samp, nsamp, st);
    return;
  }
  MfmaOut o{};
  o.S = samp;
  o.nsamp = nsamp;
  const int nch = (a.nrows + sample_chunk - 1) / sample_chunk;
  launch_mfma<MFMA_SAMPLE>(a, sample_chunk, (unsigned)((nch + 3) / 4), o, st);
}


static int device_cus() {
  static int cached[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cached[dev] = v;
  }
  return cached[dev];
}

template <int D>
static void launch_cand_persistent(const ScoreArgs& a, const MfmaOut& o, hipStream_t st) {
  const int tpg = (a.nrows + 31) / 32;
  const int64_t ntiles = (int64_t)a.B * a.Hkv * tpg;
  // stage slots per head: PS_STAGE_BYTES per wave, less 64 spare slots, over G heads x 6 bytes
  // (score bits, 16-bit position offset)
  const int S = ((PS_STAGE_BYTES / 6 - 64) / a.G) & ~1;  // even: each wave's 4-byte bits stay aligned
  const size_t lds = (size_t)4 * 32 * (D * 2 + 16) + (size_t)4 * (a.G * S + 64) * 6;
  const int fit = (int)(device_lds_limit() / lds);  // workgroups whose LDS fits one CU
  int64_t grid = (int64_t)device_cus() * std::max(1, std::min(PS_WPC, fit));
  if (grid > (ntiles + 3) / 4) grid = (ntiles + 3) / 4;
  const int M = a.M > 1 ? a.M : 1;  // the caller keeps M <= 4
  if (M > 1 && TKA_ROWS_SCAN && M * a.G <= 32) {
    // every (query, head) row of a group on one wave's tiles: the one-query scan's LDS layout with
    // R = M G rows sharing the stage
    const int R = M * a.G;
    const int S3 = ((PS_STAGE_BYTES / 6 - 64) / R) & ~1;
    const size_t lds3 = (size_t)4 * 32 * (D * 2 + 16) + (size_t)4 * (R * S3 + 64) * 6;
    const int fit3 = (int)(device_lds_limit() / lds3);
    int64_t g3 = (int64_t)device_cus() * std::max(1, std::min(PS_WPC, fit3));
    if (g3 > (ntiles + 3) / 4) g3 = (ntiles + 3) / 4;
    if (R <= 16) {
      ensure_dynamic_lds((const void*)score_cand_rows_kernel<D, 1>, lds3);
      hipLaunchKernelGGL((score_cand_rows_kernel<D, 1>), dim3((unsigned)g3), dim3(256), lds3, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, M, a.nrows, a.sb, a.sh,
                         a.sl, a.scale, ntiles, tpg, S3, o);
    } else {
      ensure_dynamic_lds((const void*)score_cand_rows_kernel<D, 2>, lds3);
      hipLaunchKernelGGL((score_cand_rows_kernel<D, 2>), dim3((unsigned)g3), dim3(256), lds3, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, M, a.nrows, a.sb, a.sh,
                         a.sl, a.scale, ntiles, tpg, S3, o);
    }
    return;
  }
  if (M > 1 && TKA_SHARED_SCAN) {
    // two tile buffers and four wave stages sized to fit SS_WPC workgroups per CU
    const size_t tiles = (size_t)2 * 32 * (D * 2 + 16);
    // stages for the scoring waves only, 16 rows each: ceil(M G / 16) blocks, two waves per block
    // (one per tile half) when there are at most two blocks
    const int ncb = (M * a.G + 15) / 16;
    const int nst = ncb <= 2 ? 2 * ncb : ncb;
    const int S2 = (int)((((size_t)device_lds_limit() / SS_WPC - tiles - 256) / (8 * (size_t)nst) - 64) / 16);
    const size_t lds2 = tiles + (size_t)nst * (16 * S2 + 64) * 8;
    int64_t g2 = (int64_t)device_cus() * SS_WPC;
    if (g2 > ntiles) g2 = ntiles;
    if (ncb <= 2) {
      ensure_dynamic_lds((const void*)score_cand_shared_kernel<D, 1>, lds2);
      hipLaunchKernelGGL((score_cand_shared_kernel<D, 1>), dim3((unsigned)g2), dim3(256), lds2, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, M, a.nrows, a.sb, a.sh, a.sl,
                         a.scale, (int)ntiles, tpg, S2, o);
    } else {
      ensure_dynamic_lds((const void*)score_cand_shared_kernel<D, 2>, lds2);
      hipLaunchKernelGGL((score_cand_shared_kernel<D, 2>), dim3((unsigned)g2), dim3(256), lds2, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, M, a.nrows, a.sb, a.sh, a.sl,
                         a.scale, (int)ntiles, tpg, S2, o);
    }
    return;
  }
  if (M == 1) {
    ensure_dynamic_lds((const void*)score_cand_persistent_kernel<D, false>, lds);
    hipLaunchKernelGGL((score_cand_persistent_kernel<D, false>), dim3((unsigned)grid), dim3(256), lds, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, 1, a.nrows, a.sb, a.sh,
                       a.sl, a.scale, ntiles, tpg, S, o);
  } else {
    ensure_dynamic_lds((const void*)score_cand_persistent_kernel<D, true>, lds);
    hipLaunchKernelGGL((score_cand_persistent_kernel<D, true>), dim3((unsigned)grid), dim3(256), lds, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, M, a.nrows, a.sb, a.sh,
                       a.sl, a.scale, ntiles, tpg, S, o);
  }
}

void launch_score_mfma_cand(const ScoreArgs& a, const MfmaOut& o, hipStream_t st) {
  switch (a.d) {
    case 64: launch_cand_persistent<64>(a, o, st); break;
    case 128: launch_cand_persistent<128>(a, o, st); break;
    default: launch_cand_persistent<256>(a, o, st); break;
  }
}

// chunk: positions per workgroup (full mode) or the sample chunk (sample mode,
// which scores the first 64 positions of each, out = [rows, nsamp])
template <int D, int RT, int MODE>
static void launch_mq_t(const ScoreArgs& a, int chunk, float* out, int nsamp, hipStream_t st) {
  const size_t lds = (size_t)4 * 32 * (D * 2 + 16);
  ensure_dynamic_lds((const void*)score_mq_kernel<D, RT, MODE>, lds);
  dim3 grid((a.nrows + chunk - 1) / chunk, a.B * a.Hkv);
  hipLaunchKernelGGL((score_mq_kernel<D, RT, MODE>), grid, dim3(256), lds, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.keys, a.Hq, a.Hkv, a.G, a.M, a.nrows, a.sb, a.sh, a.sl, a.scale, chunk, out,
                     nsamp);
}

template <int D, int MODE>
static void launch_mq_d(const ScoreArgs& a, int chunk, float* out, int nsamp, hipStream_t st) {
  const int R = a.M * a.G;
  if (R <= 16) launch_mq_t<D, 1, MODE>(a, chunk, out, nsamp, st);
  else if (R <= 32) launch_mq_t<D, 2, MODE>(a, chunk, out, nsamp, st);
  else launch_mq_t<D, 4, MODE>(a, chunk, out, nsamp, st);
}

template <int MODE>
static void launch_mq_mode(const ScoreArgs& a, int chunk, float* out, int nsamp, hipStream_t st) {
  if (a.nrows <= 0) return;
  switch (a.d) {
    case 64: launch_mq_d<64, MODE>(a, chunk, out, nsamp, st); break;
    case 128: launch_mq_d<128, MODE>(a, chunk, out, nsamp, st); break;
    default: launch_mq_d<256, MODE>(a, chunk, out, nsamp, st); break;
  }
}

void launch_score_mq(const ScoreArgs& a, hipStream_t st) {
  launch_mq_mode<MQ_FULL>(a, mfma_scan_chunk(a), a.scores, 0, st);
}

void launch_mq_counts(int32_t* krow, int64_t rows, int M, int Hq, int L, int k, hipStream_t st) {
  if (rows <= 0) return;
  const int64_t blocks = (rows + 255) / 256;
  hipLaunchKernelGGL(mq_counts_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, krow, rows,
                     M, Hq, L, k);
}

template <bool BF16, int D, int NH>
static void launch_vec_nh(const ScoreArgs& a, hipStream_t st) {
  const int htiles = (a.G + NH - 1) / NH;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int RPW = 64 / (D * ES / 16);
  const int gran = 4 * RPW * 4;
  const int chunk = pick_chunk(a.nrows, (int64_t)a.B * a.Hkv * htiles, gran, gran, 4096);
  dim3 grid((a.nrows + chunk - 1) / chunk, a.B * a.Hkv * htiles);
  hipLaunchKernelGGL((score_vec_kernel<BF16, D, NH>), grid, dim3(256), 0, st, a.q, a.keys, a.scores, a.Hq, a.Hkv,
                     a.G, a.nrows, a.sb, a.sh, a.sl, a.scale, chunk, htiles, a.q_bf16);
}

template <bool BF16, int D>
static void launch_vec_d(const ScoreArgs& a, hipStream_t st) {
  if (a.G >= 8) launch_vec_nh<BF16, D, 8>(a, st);
  else if (a.G >= 4) launch_vec_nh<BF16, D, 4>(a, st);
  else if (a.G >= 2) launch_vec_nh<BF16, D, 2>(a, st);
  else launch_vec_nh<BF16, D, 1>(a, st);
}

template <bool BF16>
static void launch_vec(const ScoreArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: launch_vec_d<BF16, 64>(a, st); break;
    case 128: launch_vec_d<BF16, 128>(a, st); break;
    default: launch_vec_d<BF16, 256>(a, st); break;
  }
}

template <int D, int NH>
static void launch_block_nh(const ScoreArgs& a, hipStream_t st) {
  using SH = BlockScoreShape<D, NH>;
  const int htiles = (a.G + NH - 1) / NH;
  const int64_t tasks = (int64_t)a.B * a.Hkv * htiles;
  int chunk = SH::ROWS;  // one pass per workgroup, unless that makes far more workgroups than the chip holds
  while (tasks * ((a.nrows + chunk - 1) / chunk) > 2048) chunk *= 2;
  dim3 grid((a.nrows + chunk - 1) / chunk, (unsigned)tasks);
  hipLaunchKernelGGL((score_block_kernel<D, NH>), grid, dim3(256), 0, st, a.q, (const float*)a.keys, a.scores, a.Hq,
                     a.Hkv, a.G, a.nrows, a.sb, a.sh, a.sl, a.scale, chunk, htiles, a.q_bf16);
}

template <int D>
static void launch_block_d(const ScoreArgs& a, hipStream_t st) {
  if (a.G > 4) launch_block_nh<D, 8>(a, st);
  else if (a.G > 2) launch_block_nh<D, 4>(a, st);
  else if (a.G > 1) launch_block_nh<D, 2>(a, st);
  else launch_block_nh<D, 1>(a, st);
}

static void launch_block(const ScoreArgs& a, hipStream_t st) {
  switch (a.d) {
    case 64: launch_block_d<64>(a, st); break;
    case 128: launch_block_d<128>(a, st); break;
    default: launch_block_d<256>(a, st); break;
  }
}

bool score_uses_mfma(int dtype_bf16, int G) { return dtype_bf16 && G >= 2 && G <= 16; }

// the full-score MFMA kernel (one query per sequence, not block means) writes a maximum per
// (chunk workgroup, wave) of each row
int score_rmax_slots(const ScoreArgs& a) {
  if (a.nrows <= 0 || a.M > 1 || a.block || !score_uses_mfma(a.bf16, a.G)) return 0;
  const int chunk = mfma_scan_chunk(a);
  return 4 * ((a.nrows + chunk - 1) / chunk);
}

void launch_score_dense(const ScoreArgs& a, hipStream_t st) {
  if (a.nrows <= 0) return;
  if (a.M > 1) {
    launch_score_mq(a, st);
    return;
  }
  if (a.block) {
    launch_block(a, st);
    return;
  }
  if (score_uses_mfma(a.bf16, a.G)) {
    MfmaOut o{};
    o.S = a.scores;
    const int chunk = mfma_scan_chunk(a);
    o.rmax = a.rmax;
    o.rmax_slots = score_rmax_slots(a);
    launch_mfma<MFMA_FULL>(a, chunk, (unsigned)((a.nrows + chunk - 1) / chunk), o, st);
  } else if (a.bf16) {
    launch_vec<true>(a, st);
  } else {
    launch_vec<false>(a, st);
  }
}

template <int DI, int NT>
static void launch_idx_t(const IndexerArgs& a, hipStream_t st) {
  const int chunk = pick_chunk(a.L, a.B, 512, 512, 8192);
  dim3 grid((a.L + chunk - 1) / chunk, a.B);
  hipLaunchKernelGGL((score_indexer_kernel<DI, NT>), grid, dim3(256), 0, st, a.qI, a.kI, a.w, a.scores, a.HI, a.L,
                     a.Lc > 0 ? a.Lc : a.L, chunk);
}

template <int DI>
static void launch_idx_d(const IndexerArgs& a, hipStream_t st) {
  if (a.HI <= 32) launch_idx_t<DI, 1>(a, st);
  else if (a.HI <= 64) launch_idx_t<DI, 2>(a, st);
  else launch_idx_t<DI, 4>(a, st);
}

void launch_score_indexer(const IndexerArgs& a, hipStream_t st) {
  if (a.dI == 64) launch_idx_d<64>(a, st);
  else launch_idx_d<128>(a, st);
}

template <bool BF16>
static void launch_bm(const BlockMeanArgs& a, hipStream_t st) {
  const int j0 = a.j0, j1 = a.j1 > 0 ? a.j1 : a.m;
  if (j1 <= j0) return;
  dim3 grid((j1 - j0 + 3) / 4, a.B * a.Hkv);
  switch (a.d) {
    case 64:
      hipLaunchKernelGGL((block_mean_kernel<BF16, 64>), grid, dim3(256), 0, st, a.K, a.means, a.Hkv, a.L, a.bsz, a.m,
                         a.sb, a.sh, a.sl, j0, j1);
      break;
    case 128:
      hipLaunchKernelGGL((block_mean_kernel<BF16, 128>), grid, dim3(256), 0, st, a.K, a.means, a.Hkv, a.L, a.bsz,
                         a.m, a.sb, a.sh, a.sl, j0, j1);
      break;
    default:
      hipLaunchKernelGGL((block_mean_kernel<BF16, 256>), grid, dim3(256), 0, st, a.K, a.means, a.Hkv, a.L, a.bsz,
                         a.m, a.sb, a.sh, a.sl, j0, j1);
      break;
  }
}

void launch_block_mean(const BlockMeanArgs& a, hipStream_t st) {
  if (a.bf16) launch_bm<true>(a, st);
  else launch_bm<false>(a, st);
}

}  // namespace tka
