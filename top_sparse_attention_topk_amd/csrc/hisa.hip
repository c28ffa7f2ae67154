// Two-level (hierarchical) selection for gfx950: "Sparse Attention
// Landscape", "Hierarchical Sparse Attention". The coarse level (block
// scores from the block means, top-K_B blocks) runs on the scoring and
// select kernels; here are the fine level's pieces: the exact scores of the
// kept blocks' tokens only, and the map from candidate slots back to
// positions.
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
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) a += __shfl_xor(a, o, kWave);
      const int64_t t = base + u * RPW + grp;
      if (t < t1 && sub == 0) crow[t] = pos[u] >= 0 ? a * scale : __int_as_float(0x7fc00000);
    }
  }
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
