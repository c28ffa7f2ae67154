// Gather - softmax - PV over the kept positions only, for gfx950.
//
// "Sparse Attention in LLM Inference", "Changes in Caching Strategy": the
// sparse layer reads only the KV entries at the positions the Top-K step
// kept, through a position index; "Computational and Memory Access
// Benefits": the attention work is O(K d) per query instead of O(L d).
//
// A task is one (b, query head) with its own kept list, or one (b, KV head)
// with the G query heads that share a kept list (indexer variant: one set per
// sequence). A task's expanded token list (block ids expand to their keys,
// plus the current block) is cut into splits, one workgroup each, which writes
// o (one split) or an (M, l, acc) partial; partials are merged in split order.
// Two kernels:
//   - gather_kernel: the logits are the selected scores (the exact variant):
//     tokens and logits into LDS, the maximum logit per head, then the V rows
//     streamed with p = exp(z - max) accumulated in fp32;
//   - gather_kv_kernel: the logits come from the K rows (the proxy-scored
//     variants): K and V slices of a row loaded together, a running softmax
//     per lane, lane groups and waves merged in a fixed order.
// Rows are read once (non-temporal 16-byte loads); every sum has a fixed order.
#include <math.h>

#include "device_common.h"
#include "internal.h"

// launch shape: workgroups the split plan aims for (a task's keys are split until the grid has
// about this many), and the K or V rows a wave has in flight per round (4 measured best: more
// rounds over short spans; at d = 128 in bf16 one round is still 16 rows of 256 B per wave)
#ifndef TKA_G_WANT
#define TKA_G_WANT 1024
#endif
#ifndef TKA_G_UNR
#define TKA_G_UNR 4
#endif

namespace tka {

struct GatherK {
  const void* q;
  const void* K;
  const void* V;
  const int32_t* idx;
  const float* sel;
  float* out;
  float* part;
  int Hq, Hkv, G, L, m;
  int64_t sb, sh, sl;
  float scale;
  int n_idx, unit, shared, nsplit, span;
  int64_t E;
  int M;  // queries per sequence (causal): task's K/V sequence is b / M, its last visible key L - M + b % M
};

// The merge of a task's split partials (PS = NH (D + 2) floats each, p at the first): for head h,
// with M the maximum of the splits' M_s and weights f_s = e^(M_s - M) (0 for an empty split),
// o = sum_s f_s acc_s / sum_s f_s l_s, accumulated in split order. wt(s) gives f_s.
template <int D, int NH, typename Wt>
__device__ __forceinline__ float merge_column(const float* __restrict__ p, int nsplit, int h, int c, Wt wt) {
  constexpr int PS = NH * (D + 2);
  float num = 0.f, den = 0.f;
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    float a[8], l[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = p[(s + u) * PS + h * D + c];
      l[u] = p[(s + u) * PS + NH * D + NH + h];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = wt(s + u);
      if (f == 0.f) continue;
      num = fmaf(f, a[u], num);
      den = fmaf(f, l[u], den);
    }
  }
  for (; s < nsplit; ++s) {
    const float f = wt(s);
    if (f == 0.f) continue;
    num = fmaf(f, p[s * PS + h * D + c], num);
    den = fmaf(f, p[s * PS + NH * D + NH + h], den);
  }
  return den > 0.f ? num / den : 0.f;
}

__device__ __forceinline__ float split_weight(float ms, float M) {
  return (M == -INFINITY || ms == -INFINITY) ? 0.f : expf(ms - M);
}

template <bool BF16, int D, int NH, bool SEL>
__global__ __launch_bounds__(256) void gather_kernel(GatherK a) {
  static_assert(SEL, "K-row logits take gather_kv_kernel");
  using U = Unpack<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = U::N;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int UNR = TKA_G_UNR;
  extern __shared__ uint4 smem_raw[];
  float* red = reinterpret_cast<float*>(smem_raw);  // [NH][D]
  float* stat = red + NH * D;                      // M[NH], l[NH], wave maxima [4][NH]
  int32_t* tok = reinterpret_cast<int32_t*>(stat + 6 * NH);
  float* lg = reinterpret_cast<float*>(tok + a.span);  // [NH][span]

  // workgroup ids remapped so that the tasks of one KV group share an XCD (and its L2)
  const unsigned lid = xcd_logical_id(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int task = (int)(lid / gridDim.x), split = (int)(lid % gridDim.x);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  int b, h0, g;
  const int32_t* list;
  const float* sl_list = nullptr;
  if (a.shared) {
    b = task / a.Hkv;
    g = task % a.Hkv;
    h0 = g * a.G;
    list = a.idx + (int64_t)b * a.n_idx;
  } else {
    b = task / a.Hq;  // a (sequence, query) pair when M > 1
    h0 = task % a.Hq;
    g = h0 / a.G;
    list = a.idx + (int64_t)task * a.n_idx;
    if (SEL) sl_list = a.sel + (int64_t)task * a.n_idx;
  }
  const int bkv = b / a.M;                 // the sequence whose K/V rows it reads
  const int lim = a.L - a.M + 1 + b % a.M;  // keys it may see (all L for one query per sequence)
  const int64_t e0 = (int64_t)split * a.span;
  const int ne = (int)max((int64_t)0, min(a.E, e0 + a.span) - e0);

  // 1. tokens (and the given logits)
  const int64_t nb = (int64_t)a.n_idx * (a.unit > 0 ? a.unit : 1);
  const bool vec = a.unit == 0 && (ne & 3) == 0 && ((reinterpret_cast<uintptr_t>(list + e0) & 15) == 0) &&
                   (!SEL || (reinterpret_cast<uintptr_t>(sl_list + e0) & 15) == 0);
  if (vec) {  // position lists: 16-byte loads, all of a thread's issued together
#pragma unroll 4
    for (int i = 4 * t; i < ne; i += 1024) {
      const int4 v = *reinterpret_cast<const int4*>(list + e0 + i);
      float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      if (SEL) z = *reinterpret_cast<const float4*>(sl_list + e0 + i);
      const int tv[4] = {v.x, v.y, v.z, v.w};
      const float zv[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int tk = (tv[c] >= 0 && tv[c] < lim) ? tv[c] : -1;
        tok[i + c] = tk;
        if (SEL) lg[i + c] = tk >= 0 ? zv[c] : -INFINITY;
      }
    }
  }
  for (int i = vec ? ne : t; i < ne; i += 256) {
    const int64_t e = e0 + i;
    int tk = -1;
    if (a.unit == 0) {
      const int v = list[e];
      tk = (v >= 0 && v < lim) ? v : -1;
    } else if (e < nb) {
      const int j = list[e / a.unit];
      if (j >= 0 && j < a.m - 1) {
        const int64_t x = (int64_t)j * a.unit + e % a.unit;
        tk = x < a.L ? (int)x : -1;
      }
    } else {
      const int64_t x = (int64_t)(a.m - 1) * a.unit + (e - nb);
      tk = x < a.L ? (int)x : -1;
    }
    tok[i] = tk;
    if (SEL) lg[i] = tk >= 0 ? sl_list[e] : -INFINITY;
  }
  __syncthreads();

  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.V) + ((int64_t)bkv * a.sb + (int64_t)g * a.sh) * ES;

  // 2. the maximum logit per head (every thread takes a strided share; waves combine through LDS)
  float* wmax = stat + 2 * NH;  // [4][NH]
  {
    float mloc[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) mloc[h] = -INFINITY;
    for (int i = t; i < ne; i += 256)
#pragma unroll
      for (int h = 0; h < NH; ++h) mloc[h] = fmaxf(mloc[h], lg[h * a.span + i]);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float m = wave_max(mloc[h]);
      if (lane == 0) wmax[w * NH + h] = m;
    }
  }
  __syncthreads();
  float mx[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h)
    mx[h] = fmaxf(fmaxf(wmax[h], wmax[NH + h]), fmaxf(wmax[2 * NH + h], wmax[3 * NH + h]));

  // 3. V gather and weighted accumulation; the weights p = exp(z - max) are formed here, and each
  //    lane group sums the weights of its own rows (the sums are combined in a fixed order below)
  float acc[NH][EPL], psum[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    psum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  for (int ib = w * RPW * UNR; ib < ne; ib += 4 * RPW * UNR) {
    uint4 raw[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = ib + u * RPW + grp;
      const int tk = i < ne ? tok[i] : -1;
      raw[u] = tk >= 0 ? ld16_stream(Vb + ((int64_t)tk * a.sl + sub * EPL) * ES) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = ib + u * RPW + grp;
      if (i < ne) {
        float vf[EPL];
        U::run(raw[u], vf);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const float z = lg[h * a.span + i];
          const float p = (mx[h] == -INFINITY) ? 0.f : expf(z - mx[h]);
          psum[h] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {  // the wave's lane groups, merged position by position
    psum[h] = cross_sum<LPR>(psum[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = cross_sum<LPR>(acc[h][e]);
  }
  // waves add their sums in a fixed order
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww && grp == 0) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float* r = red + h * D + sub * EPL + e;
          *r = (ww == 0) ? acc[h][e] : *r + acc[h][e];
        }
        if (sub == 0) stat[NH + h] = (ww == 0) ? psum[h] : stat[NH + h] + psum[h];
      }
    }
    __syncthreads();
  }
  if (t < NH) stat[t] = mx[t];
  __syncthreads();

  // 4. output or partials
  if (a.nsplit == 1) {
    for (int i = t; i < NH * D; i += 256) {
      const int h = i / D, c = i % D;
      const float l = stat[NH + h];
      a.out[((int64_t)b * a.Hq + h0 + h) * D + c] = l > 0.f ? red[i] / l : 0.f;
    }
  } else {
    float* p = a.part + ((int64_t)task * a.nsplit + split) * (NH * (D + 2));
    for (int i = t; i < NH * D; i += 256) p[i] = red[i];
    if (t < 2 * NH) p[NH * D + t] = stat[t];
  }
}

// Logits from the K rows (the proxy-scored variants): one pass that loads each
// row's K and V slices together. Every lane resolves the tokens of its own rows
// (no token staging), its lane group (LPR lanes per row) reduces the dot
// products with xor shuffles, and each lane keeps a running softmax over its
// rows in base 2 (logits y = z log2(e), weights 2^(y - m) on v_exp_f32): per
// round of UNR rows the maximum m, the mass l and acc = sum p V, rescaled by
// 2^(m_old - m) when the maximum grows. The lane groups of a wave, then the
// four waves, merge in a fixed order: the maxima first, then the rescaled
// sums. The result is the split's partial (its maximum back in natural-log
// units, as the merge expects) or, unsplit, the output.
__device__ __forceinline__ float pow2(float y) { return __builtin_amdgcn_exp2f(y); }

// byte offset of gather_kv_kernel's token array in its dynamic LDS (after the wave partials)
__host__ __device__ constexpr size_t kv_tok_offset(int NH, int D) {
  return (sizeof(float) * (4 * (size_t)NH * (D + 2) + 6 * (size_t)NH) + 15) & ~(size_t)15;
}

template <bool BF16, int D, int NH>
__global__ __launch_bounds__(256) void gather_kv_kernel(GatherK a) {
  using U = Unpack<BF16>;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = U::N;
  constexpr int LPR = D * ES / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int UNR = 4;
  constexpr int PS = NH * (D + 2);  // floats of one (m, l, acc) partial
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  extern __shared__ uint4 smem_raw[];
  float* wpart = reinterpret_cast<float*>(smem_raw);  // [4 waves][PS]: acc [NH][D], m [NH], l [NH]
  float* wfac = wpart + 4 * PS;                        // [4 waves][NH] rescale factors, M, l
  // then, 16-byte aligned: the span's tokens
  int32_t* tokl = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(smem_raw) + kv_tok_offset(NH, D));

  const unsigned lid = xcd_logical_id(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  const int task = (int)(lid / gridDim.x), split = (int)(lid % gridDim.x);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int sub = lane % LPR, grp = lane / LPR;
  int b, h0, g;
  const int32_t* list;
  if (a.shared) {
    b = task / a.Hkv;
    g = task % a.Hkv;
    h0 = g * a.G;
    list = a.idx + (int64_t)b * a.n_idx;
  } else {
    b = task / a.Hq;
    h0 = task % a.Hq;
    g = h0 / a.G;
    list = a.idx + (int64_t)task * a.n_idx;
  }
  // the query slices first: their loads overlap the token staging below
  uint4 qraw[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h)
    qraw[h] = ld16(reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)(b * a.Hq + h0 + h) * D + sub * EPL) * ES);
  const int bkv = b / a.M;
  const int lim = a.L - a.M + 1 + b % a.M;
  const int64_t e0 = (int64_t)split * a.span;
  const int ne = (int)max((int64_t)0, min(a.E, e0 + a.span) - e0);
  const int64_t nb = (int64_t)a.n_idx * (a.unit > 0 ? a.unit : 1);
  auto token = [&](int i) {  // the token of expanded entry e0 + i (-1: none)
    const int64_t e = e0 + i;
    if (a.unit == 0) {
      const int v = list[e];
      return (v >= 0 && v < lim) ? v : -1;
    }
    if (e < nb) {
      const int j = list[e / a.unit];
      if (j < 0 || j >= a.m - 1) return -1;
      const int64_t x = (int64_t)j * a.unit + e % a.unit;
      return x < a.L ? (int)x : -1;
    }
    const int64_t x = (int64_t)(a.m - 1) * a.unit + (e - nb);
    return x < a.L ? (int)x : -1;
  };

  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(a.K) + ((int64_t)bkv * a.sb + (int64_t)g * a.sh) * ES;
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.V) + ((int64_t)bkv * a.sb + (int64_t)g * a.sh) * ES;
  const float yscale = a.scale * kLog2e;
  // the span's tokens into LDS (one list read), then rounds of UNR rows per lane; with NH <= 4
  // the next round's K and V slices are in flight while the current round is reduced
#pragma unroll 4
  for (int i = t; i < ne; i += 256) tokl[i] = token(i);
  __syncthreads();
  float qf[NH][EPL];
#pragma unroll
  for (int h = 0; h < NH; ++h) U::run(qraw[h], qf[h]);
  float m[NH], l[NH], acc[NH][EPL];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  auto issue = [&](int ib, int (&tk)[UNR], uint4 (&kr)[UNR], uint4 (&vr)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = ib + u * RPW + grp;
      tk[u] = i < ne ? tokl[i] : -1;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (tk[u] >= 0) {
        const int64_t off = ((int64_t)tk[u] * a.sl + sub * EPL) * ES;
        kr[u] = ld16_stream(Kb + off);
        vr[u] = ld16_stream(Vb + off);
      }
    }
  };
  auto consume = [&](const int (&tk)[UNR], const uint4 (&kr)[UNR], const uint4 (&vr)[UNR]) {
    float y[UNR][NH];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[EPL];
      U::run(kr[u], kf);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x = fmaf(qf[h][e], kf[e], x);
        y[u][h] = x;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) y[u][h] = group_sum<LPR>(y[u][h]);  // the row's dot product
#pragma unroll
      for (int h = 0; h < NH; ++h) y[u][h] = tk[u] >= 0 ? y[u][h] * yscale : -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float mn = m[h];
#pragma unroll
      for (int u = 0; u < UNR; ++u) mn = fmaxf(mn, y[u][h]);
      if (mn == -INFINITY) continue;  // nothing seen yet
      const float sc = pow2(m[h] - mn);  // m = -inf: 0 (l and acc are still 0)
      l[h] *= sc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= sc;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float pu = pow2(y[u][h] - mn);  // y = -inf: 0
        float vf[EPL];
        U::run(vr[u], vf);
        l[h] += pu;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pu, vf[e], acc[h][e]);
      }
      m[h] = mn;
    }
  };
  constexpr int STRIDE = 4 * RPW * UNR;
  if constexpr (NH <= 4) {
    int tkc[UNR];
    uint4 krc[UNR], vrc[UNR];
    int ib = w * RPW * UNR;
    if (ib < ne) issue(ib, tkc, krc, vrc);
    for (; ib < ne; ib += STRIDE) {
      int tkn[UNR];
      uint4 krn[UNR], vrn[UNR];
      const bool more = ib + STRIDE < ne;
      if (more) issue(ib + STRIDE, tkn, krn, vrn);
      consume(tkc, krc, vrc);
      if (more) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          tkc[u] = tkn[u];
          krc[u] = krn[u];
          vrc[u] = vrn[u];
        }
      }
    }
  } else {
    for (int ib = w * RPW * UNR; ib < ne; ib += STRIDE) {
      int tk[UNR];
      uint4 kr[UNR], vr[UNR];
      issue(ib, tk, kr, vr);
      consume(tk, kr, vr);
    }
  }
  // the wave's lane groups (lanes sub, sub + LPR, ...): the maximum over the groups, each group's
  // state rescaled to it, then the sums over the groups (xor butterflies over the group index)
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const float M = cross_max<LPR>(m[h]);
    const float f = M == -INFINITY ? 0.f : pow2(m[h] - M);
    m[h] = M;
    l[h] *= f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
    l[h] = cross_sum<LPR>(l[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = cross_sum<LPR>(acc[h][e]);
  }
  if (grp == 0) {
    float* wp = wpart + w * PS;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) wp[h * D + sub * EPL + e] = acc[h][e];
      if (sub == 0) {
        wp[NH * D + h] = m[h];
        wp[NH * D + NH + h] = l[h];
      }
    }
  }
  __syncthreads();
  // the four waves: their factors 2^(m_w - M) per head, then the sums in wave order
  if (t < 4 * NH) {
    const int ww = t / NH, h = t % NH;
    float M = wpart[NH * D + h];
    for (int i = 1; i < 4; ++i) M = fmaxf(M, wpart[i * PS + NH * D + h]);
    const float mw = wpart[ww * PS + NH * D + h];
    wfac[t] = M == -INFINITY ? 0.f : pow2(mw - M);
    if (ww == 0) wfac[4 * NH + h] = M;
  }
  __syncthreads();
  for (int i = t; i < NH * D; i += 256) {
    const int h = i / D;
    float aa = 0.f, ll = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = wfac[ww * NH + h];
      aa = fmaf(f, wpart[ww * PS + i], aa);
      if (i % D == 0) ll = fmaf(f, wpart[ww * PS + NH * D + NH + h], ll);
    }
    if (a.nsplit == 1) {
      if (i % D == 0) wfac[5 * NH + h] = ll;
    } else {
      float* p = a.part + ((int64_t)task * a.nsplit + split) * PS;
      const float M = wfac[4 * NH + h];
      const float Mn = M == -INFINITY ? -INFINITY : M * kLn2;  // natural-log units for the merge
      p[i] = aa;
      if (i % D == 0) {
        p[NH * D + h] = Mn;
        p[NH * D + NH + h] = ll;
      }
    }
    if (a.nsplit == 1) wpart[i] = aa;  // wave 0's slot: this thread's own element, read no more
  }
  if (a.nsplit == 1) {
    __syncthreads();
    for (int i = t; i < NH * D; i += 256) {
      const float ll = wfac[5 * NH + i / D];
      a.out[((int64_t)b * a.Hq + h0 + i / D) * D + i % D] = ll > 0.f ? wpart[i] / ll : 0.f;
    }
  }
}

// The merge as its own launch. A workgroup per (task, head): the split weights first (to LDS), then
// thread c accumulates output column c over the splits.
constexpr int kMergeLdsSplits = 8192;
template <int D, int NH>
__global__ __launch_bounds__(256) void gather_merge_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                           int nsplit, int Hq, int Hkv, int G, int shared) {
  extern __shared__ float fw[];  // [nsplit] split weights (when nsplit <= kMergeLdsSplits)
  __shared__ float red[4];
  const int task = blockIdx.x, h = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  int b, h0;
  if (shared) {
    b = task / Hkv;
    h0 = (task % Hkv) * G;
  } else {
    b = task / Hq;
    h0 = task % Hq;
  }
  constexpr int PS = NH * (D + 2);  // floats per split partial
  const float* p = part + (int64_t)task * nsplit * PS;
  float m = -INFINITY;
  for (int s = t; s < nsplit; s += blockDim.x) m = fmaxf(m, p[s * PS + NH * D + h]);
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < (int)(blockDim.x + 63) / 64; ++i) M = fmaxf(M, red[i]);
  const bool in_lds = nsplit <= kMergeLdsSplits;
  if (in_lds)
    for (int s = t; s < nsplit; s += blockDim.x) fw[s] = split_weight(p[s * PS + NH * D + h], M);
  __syncthreads();
  for (int c = t; c < D; c += 256)
    out[((int64_t)b * Hq + h0 + h) * D + c] =
        M == -INFINITY ? 0.f
                       : merge_column<D, NH>(p, nsplit, h, c, [&](int s) {
                           return in_lds ? fw[s] : split_weight(p[s * PS + NH * D + h], M);
                         });
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
GatherPlan plan_gather(const GatherArgs& a) {
  GatherPlan pl;
  pl.heads_per_task = a.shared ? a.G : 1;
  pl.tasks = a.shared ? a.B * a.Hkv : a.B * a.Hq;
  pl.expanded = a.unit == 0 ? (int64_t)a.n_idx : (int64_t)a.n_idx * a.unit + a.unit;
  const int NH = pl.heads_per_task;
  const int span_max = NH == 1 ? 4096 : 8192 / NH;
  int64_t ns = (pl.expanded + span_max - 1) / span_max;
  const int64_t want = (TKA_G_WANT + pl.tasks - 1) / pl.tasks;
  const int64_t cap64 = (pl.expanded + 63) / 64;
  int64_t ns2 = want < cap64 ? want : cap64;
  if (ns2 > ns) ns = ns2;
  if (ns < 1) ns = 1;
  int64_t span = (pl.expanded + ns - 1) / ns;
  span = ((span + 15) / 16) * 16;
  if (span < 16) span = 16;
  ns = (pl.expanded + span - 1) / span;
  if (ns < 1) ns = 1;
  pl.nsplit = (int)ns;
  pl.span = (int)span;
  pl.ws_bytes = pl.nsplit > 1 ? sizeof(float) * (size_t)pl.tasks * pl.nsplit * NH * (a.d + 2) : 0;
  return pl;
}

template <bool BF16, int D, int NH, bool SEL>
static void launch_g(const GatherK& k, const GatherPlan& pl, hipStream_t st) {
  if constexpr (SEL) {
    const size_t lds = sizeof(float) * (NH * D + 6 * NH) + sizeof(int32_t) * pl.span + sizeof(float) * NH * pl.span;
    hipLaunchKernelGGL((gather_kernel<BF16, D, NH, true>), dim3(pl.nsplit, pl.tasks), dim3(256), lds, st, k);
  } else {
    const size_t lds = kv_tok_offset(NH, D) + sizeof(int32_t) * pl.span;
    ensure_dynamic_lds((const void*)gather_kv_kernel<BF16, D, NH>, lds);
    hipLaunchKernelGGL((gather_kv_kernel<BF16, D, NH>), dim3(pl.nsplit, pl.tasks), dim3(256), lds, st, k);
  }
  if (pl.nsplit > 1)
    hipLaunchKernelGGL((gather_merge_kernel<D, NH>), dim3(pl.tasks, NH), dim3(D < 256 ? D : 256),
                       pl.nsplit <= kMergeLdsSplits ? sizeof(float) * pl.nsplit : 0, st, k.part, k.out, pl.nsplit,
                       k.Hq, k.Hkv, k.G, k.shared);
}

template <bool BF16, int D>
static void launch_gd(const GatherK& k, const GatherPlan& pl, bool sel, hipStream_t st) {
  switch (pl.heads_per_task) {
    case 1:
      if (sel) launch_g<BF16, D, 1, true>(k, pl, st);
      else launch_g<BF16, D, 1, false>(k, pl, st);
      break;
    case 2: launch_g<BF16, D, 2, false>(k, pl, st); break;
    case 4: launch_g<BF16, D, 4, false>(k, pl, st); break;
    case 8: launch_g<BF16, D, 8, false>(k, pl, st); break;
    default: launch_g<BF16, D, 16, false>(k, pl, st); break;
  }
}

template <bool BF16>
static void launch_gb(const GatherK& k, const GatherPlan& pl, int d, bool sel, hipStream_t st) {
  switch (d) {
    case 64: launch_gd<BF16, 64>(k, pl, sel, st); break;
    case 128: launch_gd<BF16, 128>(k, pl, sel, st); break;
    default: launch_gd<BF16, 256>(k, pl, sel, st); break;
  }
}

void launch_gather(const GatherArgs& a, const GatherPlan& pl, void* ws, hipStream_t st) {
  if (pl.tasks <= 0) return;
  GatherK k;
  k.q = a.q;
  k.K = a.K;
  k.V = a.V;
  k.idx = a.idx;
  k.sel = a.sel;
  k.out = a.out;
  k.part = static_cast<float*>(ws);
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.G = a.G;
  k.L = a.L;
  k.m = a.unit > 0 ? (a.L + a.unit - 1) / a.unit : 0;
  k.sb = a.sb;
  k.sh = a.sh;
  k.sl = a.sl;
  k.scale = a.scale;
  k.n_idx = a.n_idx;
  k.unit = a.unit;
  k.shared = a.shared;
  k.nsplit = pl.nsplit;
  k.span = pl.span;
  k.E = pl.expanded;
  k.M = a.M > 1 ? a.M : 1;
  const bool sel = a.sel != nullptr;
  if (a.bf16) launch_gb<true>(k, pl, a.d, sel, st);
  else launch_gb<false>(k, pl, a.d, sel, st);
}

}  // namespace tka
