// C ABI of libtka (include/tka.h): argument checks on the host (no GPU call
// before they pass), workspace planning and the launch sequence of one
// decode step on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "internal.h"
#include "tka.h"

using namespace tka;

namespace {

thread_local char g_err[256] = "";

tka_status fail(tka_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

tka_status ok() {
  g_err[0] = 0;
  return TKA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(tka_dtype t) { return t == TKA_F32 ? 4 : (t == TKA_BF16 ? 2 : 1); }

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

int64_t n_blocks(const tka_problem* p) { return ((int64_t)p->seq_len + p->block_size - 1) / p->block_size; }
// query tokens per sequence
int64_t nqry(const tka_problem* p) { return p->n_queries > 1 ? p->n_queries : 1; }

// extent in bytes of a KV cache with the problem's strides
size_t kv_bytes(const tka_problem* p) {
  const int64_t last = (int64_t)(p->batch - 1) * p->kv_stride_b + (int64_t)(p->n_kv_heads - 1) * p->kv_stride_h +
                       (int64_t)(p->seq_len - 1) * p->kv_stride_l + p->head_dim;
  return (size_t)last * esize(p->qkv_dtype);
}

float eff_scale(const tka_problem* p) { return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim); }

// Shapes and dtypes of the attention part (q, K, V, grouping).
tka_status check_attn_shape(const tka_problem* p) {
  if (!p) return fail(TKA_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1) return fail(TKA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
  if (p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(TKA_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", p->n_q_heads, p->n_kv_heads);
  if (p->n_q_heads % p->n_kv_heads)
    return fail(TKA_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", p->n_q_heads,
                p->n_kv_heads);
  if (p->seq_len < 1) return fail(TKA_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d)", p->seq_len);
  if (p->top_k < 1) return fail(TKA_ERR_INVALID_ARG, "top_k must be >= 1 (got %d)", p->top_k);
  if (p->mode != TKA_SCORE_EXACT && p->mode != TKA_SCORE_BLOCK_MEAN && p->mode != TKA_SCORE_INDEXER &&
      p->mode != TKA_SCORE_HISA)
    return fail(TKA_ERR_INVALID_ARG, "unknown score mode %d", (int)p->mode);
  if (p->qkv_dtype != TKA_F32 && p->qkv_dtype != TKA_BF16)
    return fail(TKA_ERR_UNSUPPORTED, "qkv_dtype must be TKA_F32 or TKA_BF16 (got %d)", (int)p->qkv_dtype);
  if (p->n_queries < 0) return fail(TKA_ERR_INVALID_ARG, "n_queries must be >= 0 (got %d)", p->n_queries);
  if (p->decode_path < TKA_PATH_AUTO || p->decode_path > TKA_PATH_DENSE)
    return fail(TKA_ERR_INVALID_ARG, "decode_path %d is not TKA_PATH_AUTO, _PREFILTER or _DENSE", p->decode_path);
  if (nqry(p) > 1) {
    if (p->mode != TKA_SCORE_EXACT) return fail(TKA_ERR_INVALID_ARG, "several queries need TKA_SCORE_EXACT");
    if (p->n_queries > p->seq_len) return fail(TKA_ERR_INVALID_ARG, "n_queries above seq_len");
    if (p->qkv_dtype != TKA_BF16 || nqry(p) * (p->n_q_heads / p->n_kv_heads) > 64)
      return fail(TKA_ERR_UNSUPPORTED, "several queries are built for bf16 with n_queries * Hq/Hkv <= 64");
  }
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(TKA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", p->head_dim);
  if (p->kv_stride_l < p->head_dim || p->kv_stride_h < 0 || p->kv_stride_b < 0)
    return fail(TKA_ERR_INVALID_ARG, "bad KV strides (b=%lld h=%lld l=%lld)", (long long)p->kv_stride_b,
                (long long)p->kv_stride_h, (long long)p->kv_stride_l);
  const int64_t es = (int64_t)esize(p->qkv_dtype);
  if ((p->kv_stride_l * es) % 16 || (p->kv_stride_h * es) % 16 || (p->kv_stride_b * es) % 16)
    return fail(TKA_ERR_ALIGNMENT, "KV strides must be multiples of 16 bytes");
  const bool blocks = p->mode == TKA_SCORE_BLOCK_MEAN || p->mode == TKA_SCORE_HISA;
  if (blocks && p->block_size < 1)
    return fail(TKA_ERR_INVALID_ARG, "block_size must be >= 1 (got %d)", p->block_size);
  if (p->mode == TKA_SCORE_HISA &&
      (p->top_blocks < 1 || (int64_t)p->top_blocks * p->block_size > 0x7fffffff))
    return fail(TKA_ERR_INVALID_ARG, "top_blocks must be >= 1 with top_blocks * block_size < 2^31 (got %d)",
                p->top_blocks);
  if (p->block_capacity < 0 || (blocks && p->block_capacity > 0 && p->block_capacity < n_blocks(p)))
    return fail(TKA_ERR_INVALID_ARG, "block_capacity %d is below ceil(seq_len / block_size)", p->block_capacity);
  if (p->idx_capacity < 0 || (p->mode == TKA_SCORE_INDEXER && p->idx_capacity > 0 && p->idx_capacity < p->seq_len))
    return fail(TKA_ERR_INVALID_ARG, "idx_capacity %d is below seq_len", p->idx_capacity);
  if (p->mode == TKA_SCORE_INDEXER) {
    if (p->n_idx_heads < 1 || p->n_idx_heads > 128)
      return fail(p->n_idx_heads < 1 ? TKA_ERR_INVALID_ARG : TKA_ERR_UNSUPPORTED, "n_idx_heads %d not in [1, 128]",
                  p->n_idx_heads);
    if (p->idx_dim != 64 && p->idx_dim != 128)
      return fail(TKA_ERR_UNSUPPORTED, "idx_dim %d not built (64, 128)", p->idx_dim);
    if (p->idx_dtype != TKA_FP8_E4M3) return fail(TKA_ERR_UNSUPPORTED, "idx_dtype must be TKA_FP8_E4M3");
  }
  return TKA_OK;
}

tka_status need_ptr(const void* ptr, const char* name, bool align = true) {
  if (!ptr) return fail(TKA_ERR_INVALID_ARG, "%s is NULL", name);
  if (align && !aligned16(ptr)) return fail(TKA_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return TKA_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

tka_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TKA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// block slots per (b, KV head) in the block-mean buffer; positions per sequence in the indexer-key buffer
int64_t mean_slots(const tka_problem* p) { return p->block_capacity > 0 ? p->block_capacity : n_blocks(p); }
int64_t idx_slots(const tka_problem* p) { return p->idx_capacity > 0 ? p->idx_capacity : p->seq_len; }

ScoreArgs dense_score_args(const tka_problem* p, const void* q, const void* keys, float* scores) {
  ScoreArgs a;
  a.q = q;
  a.keys = keys;
  a.scores = scores;
  a.B = p->batch;
  a.Hq = p->n_q_heads;
  a.Hkv = p->n_kv_heads;
  a.G = p->n_q_heads / p->n_kv_heads;
  a.d = p->head_dim;
  a.q_bf16 = p->qkv_dtype == TKA_BF16;
  a.M = (int)nqry(p);
  if (p->mode == TKA_SCORE_BLOCK_MEAN || p->mode == TKA_SCORE_HISA) {
    const int64_t m = n_blocks(p), mc = mean_slots(p);
    a.nrows = p->mode == TKA_SCORE_HISA ? (int)m : (int)(m - 1);
    a.sb = (int64_t)p->n_kv_heads * mc * p->head_dim;
    a.sh = mc * p->head_dim;
    a.sl = p->head_dim;
    a.scale = 1.0f;
    a.bf16 = 0;
    a.block = 1;
  } else {
    a.nrows = p->seq_len;
    a.sb = p->kv_stride_b;
    a.sh = p->kv_stride_h;
    a.sl = p->kv_stride_l;
    a.scale = eff_scale(p);
    a.bf16 = p->qkv_dtype == TKA_BF16;
  }
  return a;
}

int64_t score_rows(const tka_problem* p) {
  return p->mode == TKA_SCORE_INDEXER ? p->batch : (int64_t)p->batch * nqry(p) * p->n_q_heads;
}

int32_t score_len(const tka_problem* p) {
  if (p->mode == TKA_SCORE_HISA) return (int32_t)n_blocks(p);  // every block competes
  return p->mode == TKA_SCORE_BLOCK_MEAN ? (int32_t)(n_blocks(p) - 1) : p->seq_len;
}

size_t q_bytes(const tka_problem* p) {
  if (p->mode == TKA_SCORE_INDEXER) return (size_t)p->batch * p->n_idx_heads * p->idx_dim;
  return (size_t)p->batch * nqry(p) * p->n_q_heads * p->head_dim * esize(p->qkv_dtype);
}

size_t proxy_bytes(const tka_problem* p) {
  if (p->mode == TKA_SCORE_BLOCK_MEAN || p->mode == TKA_SCORE_HISA)
    return sizeof(float) * (size_t)p->batch * p->n_kv_heads * mean_slots(p) * p->head_dim;
  if (p->mode == TKA_SCORE_INDEXER) return (size_t)p->batch * idx_slots(p) * p->idx_dim;
  return kv_bytes(p);
}

tka_status check_score_call(const tka_problem* p, const void* q, const void* keys, const float* w,
                            const float* scores) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if ((s = need_ptr(q, "q")) || (s = need_ptr(keys, "keys")) || (s = need_ptr(scores, "scores", false))) return s;
  if (reinterpret_cast<uintptr_t>(scores) & 3) return fail(TKA_ERR_ALIGNMENT, "scores is not 4-byte aligned");
  if (p->mode == TKA_SCORE_INDEXER) {
    if ((s = need_ptr(w, "idx_w", false))) return s;
    if (reinterpret_cast<uintptr_t>(w) & 3) return fail(TKA_ERR_ALIGNMENT, "idx_w is not 4-byte aligned");
  } else if (w) {
    return fail(TKA_ERR_INVALID_ARG, "idx_w must be NULL unless mode is TKA_SCORE_INDEXER");
  }
  const Range so = span_of(scores, sizeof(float) * (size_t)score_rows(p) * score_len(p));
  if (overlap(so, span_of(q, q_bytes(p))) || overlap(so, span_of(keys, proxy_bytes(p))) ||
      (w && overlap(so, span_of(w, sizeof(float) * (size_t)p->batch * p->n_idx_heads))))
    return fail(TKA_ERR_INVALID_ARG, "scores overlaps an input");
  return TKA_OK;
}

IndexerArgs indexer_args(const tka_problem* p, const void* q, const void* keys, const float* w, float* scores) {
  IndexerArgs a;
  a.qI = static_cast<const uint8_t*>(q);
  a.kI = static_cast<const uint8_t*>(keys);
  a.w = w;
  a.scores = scores;
  a.B = p->batch;
  a.HI = p->n_idx_heads;
  a.dI = p->idx_dim;
  a.L = p->seq_len;
  a.Lc = (int)idx_slots(p);
  return a;
}

void run_score(const tka_problem* p, const void* q, const void* keys, const float* w, float* scores,
               hipStream_t st) {
  if (p->mode == TKA_SCORE_INDEXER) {
    launch_score_indexer(indexer_args(p, q, keys, w, scores), st);
  } else {
    launch_score_dense(dense_score_args(p, q, keys, scores), st);
  }
}

tka_status check_select_args(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride, int32_t k,
                             const int32_t* idx_out, const float* sel) {
  if (n_rows < 0) return fail(TKA_ERR_INVALID_ARG, "n_rows must be >= 0");
  if (row_len < 0) return fail(TKA_ERR_INVALID_ARG, "row_len must be >= 0");
  if (k < 1) return fail(TKA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (n_rows > 0x7fffffff) return fail(TKA_ERR_UNSUPPORTED, "n_rows above 2^31-1");
  if (row_stride < row_len) return fail(TKA_ERR_INVALID_ARG, "row_stride %lld < row_len %d", (long long)row_stride,
                                        row_len);
  if (n_rows == 0) return TKA_OK;
  if (!scores && row_len > 0) return fail(TKA_ERR_INVALID_ARG, "scores is NULL");
  if (!idx_out) return fail(TKA_ERR_INVALID_ARG, "idx_out is NULL");
  if ((reinterpret_cast<uintptr_t>(scores) & 3) || (reinterpret_cast<uintptr_t>(idx_out) & 3) ||
      (reinterpret_cast<uintptr_t>(sel) & 3))
    return fail(TKA_ERR_ALIGNMENT, "scores, idx_out and sel_scores_out must be 4-byte aligned");
  const Range in = span_of(scores, sizeof(float) * (size_t)((n_rows - 1) * row_stride + row_len));
  const Range io = span_of(idx_out, sizeof(int32_t) * (size_t)n_rows * k);
  if (overlap(in, io)) return fail(TKA_ERR_INVALID_ARG, "idx_out overlaps scores");
  if (sel) {
    const Range so = span_of(sel, sizeof(float) * (size_t)n_rows * k);
    if (overlap(in, so) || overlap(io, so)) return fail(TKA_ERR_INVALID_ARG, "sel_scores_out overlaps");
  }
  return TKA_OK;
}

GatherArgs gather_args(const tka_problem* p, const void* q, const void* K, const void* V, const int32_t* idx,
                       int32_t n_idx, int32_t unit, int32_t shared, const float* sel, float* out) {
  GatherArgs a;
  a.q = q;
  a.K = K;
  a.V = V;
  a.idx = idx;
  a.sel = sel;
  a.out = out;
  a.B = (int)(p->batch * nqry(p));  // (sequence, query) pairs
  a.M = (int)nqry(p);
  a.Hq = p->n_q_heads;
  a.Hkv = p->n_kv_heads;
  a.G = p->n_q_heads / p->n_kv_heads;
  a.d = p->head_dim;
  a.L = p->seq_len;
  a.sb = p->kv_stride_b;
  a.sh = p->kv_stride_h;
  a.sl = p->kv_stride_l;
  a.scale = eff_scale(p);
  a.bf16 = p->qkv_dtype == TKA_BF16;
  a.n_idx = n_idx;
  a.unit = unit;
  a.shared = shared ? 1 : 0;
  return a;
}

tka_status check_gather_shape(const tka_problem* p, int32_t n_idx, int32_t unit, int32_t shared,
                              const float* sel) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (n_idx < 1) return fail(TKA_ERR_INVALID_ARG, "n_idx must be >= 1 (got %d)", n_idx);
  if (unit < 0) return fail(TKA_ERR_INVALID_ARG, "idx_unit must be >= 0 (got %d)", unit);
  if ((int64_t)n_idx * (unit > 0 ? unit : 1) + unit > 0x7fffffffLL)
    return fail(TKA_ERR_UNSUPPORTED, "expanded index list too long");
  const int G = p->n_q_heads / p->n_kv_heads;
  if (shared && G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(TKA_ERR_UNSUPPORTED, "shared index lists need Hq/Hkv in {1,2,4,8,16} (got %d)", G);
  if (sel && (shared || unit != 0))
    return fail(TKA_ERR_INVALID_ARG, "sel_scores needs per-head token lists (shared 0, idx_unit 0)");
  if (nqry(p) > 1 && (shared || unit != 0))
    return fail(TKA_ERR_INVALID_ARG, "several queries take per-head token lists (shared 0, idx_unit 0)");
  return TKA_OK;
}

size_t attn_q_bytes(const tka_problem* p) {
  return (size_t)p->batch * nqry(p) * p->n_q_heads * p->head_dim * esize(p->qkv_dtype);
}

size_t out_bytes(const tka_problem* p) {
  return sizeof(float) * (size_t)p->batch * nqry(p) * p->n_q_heads * p->head_dim;
}

// q, K, V, out pointers of the attention part and out's overlap with them
tka_status check_attn_ptrs(const tka_problem* p, const void* q, const void* K, const void* V, const float* out) {
  tka_status s;
  if ((s = need_ptr(q, "q")) || (s = need_ptr(K, "k_cache")) || (s = need_ptr(V, "v_cache")) ||
      (s = need_ptr(out, "out")))
    return s;
  const Range o = span_of(out, out_bytes(p));
  if (overlap(o, span_of(q, attn_q_bytes(p))) || overlap(o, span_of(K, kv_bytes(p))) ||
      overlap(o, span_of(V, kv_bytes(p))))
    return fail(TKA_ERR_INVALID_ARG, "out overlaps an input");
  return TKA_OK;
}

tka_status check_gather_ptrs(const tka_problem* p, const void* q, const void* K, const void* V, const int32_t* idx,
                             int32_t n_idx, int32_t shared, const float* sel, const float* out) {
  tka_status s;
  if ((s = check_attn_ptrs(p, q, K, V, out)) || (s = need_ptr(idx, "idx", false))) return s;
  if ((reinterpret_cast<uintptr_t>(idx) & 3) || (reinterpret_cast<uintptr_t>(sel) & 3))
    return fail(TKA_ERR_ALIGNMENT, "idx and sel_scores must be 4-byte aligned");
  const Range o = span_of(out, out_bytes(p));
  const size_t lists = shared ? (size_t)p->batch : (size_t)p->batch * p->n_q_heads;
  if (overlap(o, span_of(idx, sizeof(int32_t) * lists * n_idx)) ||
      (sel && overlap(o, span_of(sel, sizeof(float) * lists * n_idx))))
    return fail(TKA_ERR_INVALID_ARG, "out overlaps an input");
  return TKA_OK;
}

// ---- fused exact step: candidate prefilter plan ----
// Used for the bf16 MFMA scan when the kept fraction is small (k' <= L/8) and
// the row is long. Samples are the first 64 positions of every sample chunk,
// the chunk halved (down to 128) until E = k' nsamp / L, the samples expected
// among the k' largest keys, reaches about 57. The threshold is the r-th
// largest sample with r = ceil(E + 4.5 sqrt(E)) + 2: for exchangeable scores
// the k'-th largest key falls below it (a shortfall) only a few times in a
// million rows, and about r L / nsamp keys are expected at or above it (C3:
// E = 64, r = 102, 1.6 k'). The list capacity covers that count plus four
// standard deviations of it, L (r + 4 sqrt(r)) / nsamp, and at least 3 k'.
// A shortfall or an overflow is detected and repaired by a full rescore of
// the row's group anyway.
struct PrefilterPlan {
  bool on;
  int sample_chunk, nsamp, r, capg;
};

int64_t sample_count(int64_t L, int64_t sc) {
  const int64_t nch = (L + sc - 1) / sc;
  const int64_t last = L - (nch - 1) * sc;
  return 64 * (nch - 1) + (last < 64 ? last : 64);
}

PrefilterPlan prefilter_plan(const tka_problem* p) {
  PrefilterPlan pf{};
  const int G = p->n_q_heads / p->n_kv_heads;
  if (p->mode != TKA_SCORE_EXACT || p->qkv_dtype != TKA_BF16 || !score_uses_mfma(1, G)) return pf;
  const int64_t L = p->seq_len, kk = p->top_k < p->seq_len ? p->top_k : p->seq_len;
  // automatic: the prefilter from 2^22 scores (C2's 32 rows of 32K, 1M scores: 0.070 ms against
  // 0.0645 for the dense composition; C3's 134M: 0.90 against 1.27)
  if (p->decode_path == TKA_PATH_DENSE) return pf;
  if (p->decode_path == TKA_PATH_AUTO && (int64_t)p->batch * nqry(p) * p->n_q_heads * L < (int64_t(1) << 22)) return pf;
  // several queries per sequence: up to 4 (the scan's waves take one query each on shared tiles)
  if (L < 8192 || L > 262144 || kk * 8 > L || nqry(p) > 4) return pf;
  int64_t sc = 4096;
  while (sc > 128 && 7 * kk * sample_count(L, sc) < 4 * 100 * L) sc >>= 1;
  pf.sample_chunk = (int)sc;
  pf.nsamp = (int)sample_count(L, sc);
  // r: the samples expected among the k' largest, E = k' nsamp / L, plus 4.5 standard deviations
  // of that count (and 2): the k'-th largest key is below T only a few times in a million rows
  const double E = (double)kk * pf.nsamp / (double)L;
  pf.r = (int)std::ceil(E + 4.5 * std::sqrt(E)) + 2;
  if (pf.r > pf.nsamp) pf.r = pf.nsamp;
  if (pf.r < 1) pf.r = 1;
  const double expect = ((double)pf.r + 4.0 * std::sqrt((double)pf.r)) * (double)L / (double)pf.nsamp;
  pf.capg = (int)std::max<double>(3.0 * (double)kk, std::ceil(expect));
  // the threshold and finish kernels hold the samples and the candidates in registers
  if (pf.nsamp > 8192 || pf.capg > 12288) return PrefilterPlan{};
  pf.on = true;
  return pf;
}

// ---- fused step: workspace layout ----
struct DecodeLayout {
  size_t scores, sel_ws, idx, selv, gather_ws, krow, total;
  size_t samp, T, cnt, row_flag, group_flag, cpair;
  size_t icand;  // the indexer select's candidates
  int64_t rows;
  int32_t len;
  int32_t k;
  GatherPlan gp;
  PrefilterPlan pf;
  IndexerCandPlan ic;
  int unit, shared;
};

DecodeLayout decode_layout(const tka_problem* p) {
  DecodeLayout d;
  d.rows = score_rows(p);
  d.len = score_len(p);
  d.k = p->top_k;
  d.unit = p->mode == TKA_SCORE_BLOCK_MEAN ? p->block_size : 0;
  d.shared = p->mode == TKA_SCORE_INDEXER;
  d.pf = prefilter_plan(p);
  size_t o = 0;
  // the score array, or with the prefilter the repair kernel's bounded score slots
  d.scores = o;
  if (d.pf.on)
    o += al256(repair_slot_bytes((int64_t)p->batch * p->n_kv_heads, (int)nqry(p) * (p->n_q_heads / p->n_kv_heads),
                                 p->seq_len));
  else
    o += al256(sizeof(float) * (size_t)d.rows * (d.len > 0 ? d.len : 1));
  d.ic = d.shared ? indexer_cand_plan(p->seq_len, d.k) : IndexerCandPlan{};
  d.sel_ws = o;
  if (!d.ic.on && !d.pf.on) o += al256(select_workspace_bytes(d.rows, d.len, d.k));  // the row select's scratch
  d.idx = o;
  o += al256(sizeof(int32_t) * (size_t)d.rows * d.k);
  d.selv = o;
  o += al256(sizeof(float) * (size_t)d.rows * d.k);
  GatherArgs ga = gather_args(p, nullptr, nullptr, nullptr, nullptr, d.k, d.unit, d.shared, nullptr, nullptr);
  d.gp = plan_gather(ga);
  d.gather_ws = o;
  o += al256(d.gp.ws_bytes);
  d.krow = o;  // several queries without the prefilter: each row's count
  if (nqry(p) > 1 && !d.pf.on) o += al256(sizeof(int32_t) * (size_t)d.rows);
  if (d.pf.on) {
    const size_t R = (size_t)d.rows;
    d.samp = o;
    o += al256(sizeof(float) * R * d.pf.nsamp);
    d.T = o;
    o += al256(sizeof(uint32_t) * R);
    d.cnt = o;
    o += al256(sizeof(uint32_t) * R);
    d.row_flag = o;
    o += al256(sizeof(uint32_t) * R);
    d.group_flag = o;
    o += al256(sizeof(uint32_t) * (size_t)p->batch * p->n_kv_heads);
    d.cpair = o;  // (score bits, position) pairs
    o += al256(sizeof(uint2) * R * d.pf.capg);
  }
  d.icand = o;
  o += al256(indexer_cand_bytes(p->batch, d.ic));
  d.total = o;
  return d;
}

}  // namespace

extern "C" {

int32_t tka_abi_version(void) { return TKA_ABI_VERSION; }

const char* tka_last_error(void) { return g_err; }

const char* tka_status_str(tka_status s) {
  switch (s) {
    case TKA_OK: return "TKA_OK";
    case TKA_ERR_INVALID_ARG: return "TKA_ERR_INVALID_ARG";
    case TKA_ERR_UNSUPPORTED: return "TKA_ERR_UNSUPPORTED";
    case TKA_ERR_WORKSPACE: return "TKA_ERR_WORKSPACE";
    case TKA_ERR_ALIGNMENT: return "TKA_ERR_ALIGNMENT";
    case TKA_ERR_HIP: return "TKA_ERR_HIP";
  }
  return "TKA_UNKNOWN_STATUS";
}

tka_status topk_attn_score(const tka_problem* p, const void* q, const void* keys, const float* idx_w, float* scores,
                           void* stream) {
  tka_status s = check_score_call(p, q, keys, idx_w, scores);
  if (s) return s;
  if (score_len(p) <= 0) return ok();
  run_score(p, q, keys, idx_w, scores, as_stream(stream));
  return launched("topk_attn_score");
}

tka_status topk_attn_score_threshold(const tka_problem* p, const void* q, const void* k_cache,
                                     const float* thresholds, uint32_t* counts, float* cand_scores, int32_t* cand_pos,
                                     int32_t capacity, void* stream) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (nqry(p) > 4) return fail(TKA_ERR_UNSUPPORTED, "the thresholded scan takes at most 4 queries per sequence");
  const int G = p->n_q_heads / p->n_kv_heads;
  if (p->mode != TKA_SCORE_EXACT) return fail(TKA_ERR_INVALID_ARG, "mode must be TKA_SCORE_EXACT");
  if (p->qkv_dtype != TKA_BF16 || !score_uses_mfma(1, G))
    return fail(TKA_ERR_UNSUPPORTED, "thresholded scan needs bf16 caches and 2 <= Hq/Hkv <= 16");
  if (capacity < 1) return fail(TKA_ERR_INVALID_ARG, "capacity must be >= 1 (got %d)", capacity);
  if ((s = need_ptr(q, "q")) || (s = need_ptr(k_cache, "k_cache")) ||
      (s = need_ptr(thresholds, "thresholds", false)) || (s = need_ptr(counts, "counts", false)) ||
      (s = need_ptr(cand_scores, "cand_scores", false)) || (s = need_ptr(cand_pos, "cand_pos", false)))
    return s;
  if ((reinterpret_cast<uintptr_t>(thresholds) | reinterpret_cast<uintptr_t>(counts) |
       reinterpret_cast<uintptr_t>(cand_scores) | reinterpret_cast<uintptr_t>(cand_pos)) & 3)
    return fail(TKA_ERR_ALIGNMENT, "thresholds, counts and candidate arrays must be 4-byte aligned");
  const size_t rows = (size_t)p->batch * nqry(p) * p->n_q_heads;
  const Range co = span_of(counts, sizeof(uint32_t) * rows);
  const Range cs = span_of(cand_scores, sizeof(float) * rows * (size_t)capacity);
  const Range cp = span_of(cand_pos, sizeof(int32_t) * rows * (size_t)capacity);
  const Range ins[3] = {span_of(q, attn_q_bytes(p)), span_of(k_cache, kv_bytes(p)),
                        span_of(thresholds, sizeof(float) * rows)};
  for (const Range& in : ins)
    if (overlap(in, co) || overlap(in, cs) || overlap(in, cp))
      return fail(TKA_ERR_INVALID_ARG, "an output overlaps an input");
  if (overlap(co, cs) || overlap(co, cp) || overlap(cs, cp)) return fail(TKA_ERR_INVALID_ARG, "outputs overlap");
  MfmaOut mo{};
  mo.T = thresholds;
  mo.cnt = counts;
  mo.cbits = reinterpret_cast<uint32_t*>(cand_scores);
  mo.cpos = cand_pos;
  mo.capg = capacity;
  launch_score_mfma_cand(dense_score_args(p, q, k_cache, nullptr), mo, as_stream(stream));
  return launched("topk_attn_score_threshold");
}

tka_status topk_select_workspace_size(int64_t n_rows, int32_t row_len, int32_t k, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  if (n_rows < 0 || row_len < 0 || k < 1) return fail(TKA_ERR_INVALID_ARG, "bad select shape");
  *bytes = select_workspace_bytes(n_rows, row_len, k);
  return ok();
}

tka_status topk_select(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride, int32_t k,
                       int32_t* idx_out, float* sel_scores_out, void* ws, size_t ws_bytes, void* stream) {
  tka_status s = check_select_args(scores, n_rows, row_len, row_stride, k, idx_out, sel_scores_out);
  if (!s && !select_len_supported(n_rows, row_len))
    s = fail(TKA_ERR_UNSUPPORTED, "row_len %d too long for fewer than 128 rows (at most about 12M)", row_len);
  if (s) return s;
  const size_t need = select_workspace_bytes(n_rows, row_len, k);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TKA_ERR_WORKSPACE, "select needs %zu workspace bytes (got %zu)", need, ws_bytes);
  if (need > 0 && !aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (n_rows == 0) return ok();
  SelectArgs a{scores, n_rows, row_len, row_stride, k, idx_out, sel_scores_out};
  launch_select(a, ws, as_stream(stream));
  return launched("topk_select");
}

// ---- certified adaptive k ----
}  // extern "C"

namespace {
struct AdaptiveScratch {
  size_t W, M, flag, total;
};
AdaptiveScratch adaptive_scratch(int64_t n_rows) {
  AdaptiveScratch a;
  a.W = 0;
  a.M = al256(sizeof(uint64_t) * (size_t)n_rows);
  a.flag = a.M + al256(sizeof(float) * (size_t)n_rows);
  a.total = a.flag + al256(sizeof(uint32_t) * (size_t)n_rows);
  return a;
}
tka_status check_adaptive_args(float eps, int32_t k_min, int64_t n_rows, const int32_t* k_out, const float* tau_out,
                               Range scores_in, Range idx_range) {
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(TKA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (k_min < 0) return fail(TKA_ERR_INVALID_ARG, "k_min must be >= 0");
  if (n_rows == 0) return TKA_OK;
  if (!k_out || !tau_out) return fail(TKA_ERR_INVALID_ARG, "k_out and tau_out must not be NULL");
  if ((reinterpret_cast<uintptr_t>(k_out) & 3) || (reinterpret_cast<uintptr_t>(tau_out) & 3))
    return fail(TKA_ERR_ALIGNMENT, "k_out and tau_out must be 4-byte aligned");
  const Range ko = span_of(k_out, sizeof(int32_t) * (size_t)n_rows);
  const Range to = span_of(tau_out, sizeof(float) * (size_t)n_rows);
  if (overlap(ko, to) || overlap(ko, scores_in) || overlap(to, scores_in) || overlap(ko, idx_range) ||
      overlap(to, idx_range))
    return fail(TKA_ERR_INVALID_ARG, "k_out or tau_out overlaps another buffer");
  return TKA_OK;
}
}  // namespace

extern "C" {

tka_status topk_select_adaptive_workspace_size(int64_t n_rows, int32_t row_len, int32_t k_max, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  if (n_rows < 0 || row_len < 0 || k_max < 1) return fail(TKA_ERR_INVALID_ARG, "bad n_rows, row_len or k_max");
  *bytes = adaptive_scratch(n_rows).total;
  return ok();
}

tka_status topk_select_adaptive(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride, float eps,
                                int32_t k_min, int32_t k_max, int32_t* idx_out, int32_t* k_out, float* tau_out,
                                float* sel_scores_out, void* ws, size_t ws_bytes, void* stream) {
  tka_status s = check_select_args(scores, n_rows, row_len, row_stride, k_max, idx_out, sel_scores_out);
  if (s) return s;
  const Range in = n_rows ? span_of(scores, sizeof(float) * (size_t)((n_rows - 1) * row_stride + row_len)) : Range{};
  const Range io = n_rows ? span_of(idx_out, sizeof(int32_t) * (size_t)n_rows * k_max) : Range{};
  if ((s = check_adaptive_args(eps, k_min, n_rows, k_out, tau_out, in, io))) return s;
  const AdaptiveScratch sc = adaptive_scratch(n_rows);
  if (!ws || ws_bytes < sc.total)
    return fail(TKA_ERR_WORKSPACE, "adaptive select needs %zu workspace bytes (got %zu)", sc.total, ws_bytes);
  if (!aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (n_rows == 0) return ok();
  char* base = static_cast<char*>(ws);
  SelectArgs a{scores, n_rows, row_len, row_stride, k_max, idx_out, sel_scores_out};
  launch_select_adaptive(a, eps, k_min, k_out, reinterpret_cast<uint64_t*>(base + sc.W),
                         reinterpret_cast<float*>(base + sc.M), reinterpret_cast<uint32_t*>(base + sc.flag), tau_out,
                         as_stream(stream));
  return launched("topk_select_adaptive");
}

tka_status sparse_attn_gather_workspace_size(const tka_problem* p, int32_t n_idx, int32_t idx_unit,
                                             int32_t shared_across_heads, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  tka_status s = check_gather_shape(p, n_idx, idx_unit, shared_across_heads, nullptr);
  if (s) return s;
  GatherArgs ga = gather_args(p, nullptr, nullptr, nullptr, nullptr, n_idx, idx_unit, shared_across_heads, nullptr,
                              nullptr);
  *bytes = plan_gather(ga).ws_bytes;
  return ok();
}

tka_status sparse_attn_gather(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int32_t n_idx, int32_t idx_unit, int32_t shared_across_heads,
                              const float* sel_scores, float* out, void* ws, size_t ws_bytes, void* stream) {
  tka_status s = check_gather_shape(p, n_idx, idx_unit, shared_across_heads, sel_scores);
  if (s) return s;
  if ((s = check_gather_ptrs(p, q, k_cache, v_cache, idx, n_idx, shared_across_heads, sel_scores, out))) return s;
  GatherArgs ga =
      gather_args(p, q, k_cache, v_cache, idx, n_idx, idx_unit, shared_across_heads, sel_scores, out);
  const GatherPlan pl = plan_gather(ga);
  if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes))
    return fail(TKA_ERR_WORKSPACE, "gather needs %zu workspace bytes (got %zu)", pl.ws_bytes, ws_bytes);
  if (pl.ws_bytes > 0 && !aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  launch_gather(ga, pl, ws, as_stream(stream));
  return launched("sparse_attn_gather");
}

tka_status topk_decode_workspace_size(const tka_problem* p, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  tka_status s = check_attn_shape(p);
  if (s) return s;
  *bytes = decode_layout(p).total;
  return ok();
}

}  // extern "C"

namespace {
// every host-side check of a fused step (nothing touches the GPU); d receives the step's layout
tka_status check_decode_call(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                             const void* proxy_keys, const void* q_idx, const float* idx_w, const float* out,
                             const int32_t* idx_out, DecodeLayout& d) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (p->mode == TKA_SCORE_HISA) return fail(TKA_ERR_INVALID_ARG, "TKA_SCORE_HISA runs through topk_hisa_decode");
  const int shared = p->mode == TKA_SCORE_INDEXER ? 1 : 0;
  if ((s = check_gather_shape(p, p->top_k, p->mode == TKA_SCORE_BLOCK_MEAN ? p->block_size : 0, shared, nullptr)))
    return s;
  if (p->mode == TKA_SCORE_EXACT) {
    if (proxy_keys || q_idx || idx_w)
      return fail(TKA_ERR_INVALID_ARG, "proxy_keys, q_idx and idx_w must be NULL for TKA_SCORE_EXACT");
  } else if (p->mode == TKA_SCORE_BLOCK_MEAN) {
    if ((s = need_ptr(proxy_keys, "proxy_keys (block means)"))) return s;
    if (q_idx || idx_w) return fail(TKA_ERR_INVALID_ARG, "q_idx and idx_w must be NULL for TKA_SCORE_BLOCK_MEAN");
  } else {
    if ((s = need_ptr(proxy_keys, "proxy_keys (indexer keys)")) || (s = need_ptr(q_idx, "q_idx")) ||
        (s = need_ptr(idx_w, "idx_w", false)))
      return s;
    if (reinterpret_cast<uintptr_t>(idx_w) & 3) return fail(TKA_ERR_ALIGNMENT, "idx_w is not 4-byte aligned");
  }
  d = decode_layout(p);
  if (!select_len_supported(d.rows, d.len))
    return fail(TKA_ERR_UNSUPPORTED, "seq_len %d too long for %lld selected rows (at most about 12M)", d.len,
                (long long)d.rows);
  if ((s = check_attn_ptrs(p, q, k_cache, v_cache, out))) return s;
  const Range o = span_of(out, out_bytes(p));
  if (proxy_keys && overlap(o, span_of(proxy_keys, proxy_bytes(p))))
    return fail(TKA_ERR_INVALID_ARG, "out overlaps proxy_keys");
  if (q_idx && overlap(o, span_of(q_idx, q_bytes(p)))) return fail(TKA_ERR_INVALID_ARG, "out overlaps q_idx");
  if (idx_w && overlap(o, span_of(idx_w, sizeof(float) * (size_t)p->batch * p->n_idx_heads)))
    return fail(TKA_ERR_INVALID_ARG, "out overlaps idx_w");
  if (idx_out) {
    if (reinterpret_cast<uintptr_t>(idx_out) & 3) return fail(TKA_ERR_ALIGNMENT, "idx_out is not 4-byte aligned");
    const Range io = span_of(idx_out, sizeof(int32_t) * (size_t)d.rows * d.k);
    if (overlap(io, o) || overlap(io, span_of(k_cache, kv_bytes(p))) || overlap(io, span_of(v_cache, kv_bytes(p))) ||
        overlap(io, span_of(q, attn_q_bytes(p))) ||
        (proxy_keys && overlap(io, span_of(proxy_keys, proxy_bytes(p)))))
      return fail(TKA_ERR_INVALID_ARG, "idx_out overlaps another buffer");
  }
  return TKA_OK;
}

// the launches of a fused step on stream st, its scratch at base (d.total bytes, 256-byte aligned)
tka_status run_decode(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                      const void* proxy_keys, const void* q_idx, const float* idx_w, float* out, int32_t* idx_out,
                      const DecodeLayout& d, char* base, hipStream_t st) {
  float* scores = reinterpret_cast<float*>(base + d.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + d.idx);
  float* selv = reinterpret_cast<float*>(base + d.selv);
  const bool exact = p->mode == TKA_SCORE_EXACT;

  SelectArgs sa{scores, d.rows, d.len, (int64_t)d.len, d.k, idx, exact ? selv : nullptr};
  if (d.pf.on) {
    // 1+2. sampled threshold, candidate scan, exact select on the candidates;
    // rows whose candidates cannot hold the answer are rescored in full
    const ScoreArgs sc = dense_score_args(p, q, k_cache, scores);
    float* samp = reinterpret_cast<float*>(base + d.samp);
    float* T = reinterpret_cast<float*>(base + d.T);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(base + d.cnt);
    uint32_t* row_flag = reinterpret_cast<uint32_t*>(base + d.row_flag);
    uint32_t* group_flag = reinterpret_cast<uint32_t*>(base + d.group_flag);
    uint2* cpair = reinterpret_cast<uint2*>(base + d.cpair);
    const int G = p->n_q_heads / p->n_kv_heads;
    launch_score_mfma_sample(sc, d.pf.sample_chunk, d.pf.nsamp, samp, st);
    const int M = (int)nqry(p);
    launch_prefilter_threshold(samp, d.rows, d.pf.nsamp, d.pf.r, T, cnt, row_flag, group_flag, G, p->n_q_heads, M,
                               st);
    MfmaOut mo{};
    mo.T = T;
    mo.cnt = cnt;
    mo.cpair = cpair;
    mo.capg = d.pf.capg;
    launch_score_mfma_cand(sc, mo, st);
    launch_prefilter_finish(cpair, cnt, T, d.pf.capg, d.rows, d.len, d.k, G, p->n_q_heads, M, idx, selv,
                            row_flag, group_flag, st);
    // flagged rows: their groups' exact scores in bounded slots, then the row select (query t of
    // several keeps min(k, L - M + t + 1))
    RepairArgs ra;
    ra.q = q;
    ra.K = k_cache;
    ra.B = p->batch;
    ra.Hq = p->n_q_heads;
    ra.Hkv = p->n_kv_heads;
    ra.G = G;
    ra.M = M;
    ra.d = p->head_dim;
    ra.L = p->seq_len;
    ra.k = d.k;
    ra.sb = p->kv_stride_b;
    ra.sh = p->kv_stride_h;
    ra.sl = p->kv_stride_l;
    ra.scale = eff_scale(p);
    ra.group_flag = group_flag;
    ra.row_flag = row_flag;
    ra.slots = scores;
    ra.idx = idx;
    ra.sel = selv;
    launch_prefilter_repair(ra, st);
  } else if (d.ic.on) {
    // 1+2. indexer scores with each chunk's candidates, then the select among the candidates
    launch_indexer_select(indexer_args(p, q_idx, proxy_keys, idx_w, scores), d.ic, d.k, base + d.icand, idx,
                          nullptr, st);
  } else {
    // 1. score
    if (p->mode == TKA_SCORE_INDEXER) run_score(p, q_idx, proxy_keys, idx_w, scores, st);
    else if (d.len > 0) run_score(p, q, exact ? k_cache : proxy_keys, nullptr, scores, st);
    // 2. select (several queries: query t keeps min(k, L - M + t + 1) of its visible keys)
    if (nqry(p) > 1) {
      int32_t* krow = reinterpret_cast<int32_t*>(base + d.krow);
      launch_mq_counts(krow, d.rows, (int)nqry(p), p->n_q_heads, p->seq_len, d.k, st);
      launch_select_rows_counts(sa, krow, st);
    } else {
      launch_select(sa, base + d.sel_ws, st);
    }
  }
  // 3. gather
  GatherArgs ga = gather_args(p, q, k_cache, v_cache, idx, d.k, d.unit, d.shared, exact ? selv : nullptr, out);
  launch_gather(ga, d.gp, base + d.gather_ws, st);
  return launched("topk_decode");
}

}  // namespace

extern "C" {

tka_status topk_decode(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                       const void* proxy_keys, const void* q_idx, const float* idx_w, float* out, int32_t* idx_out,
                       void* ws, size_t ws_bytes, void* stream) {
  DecodeLayout d;
  tka_status s = check_decode_call(p, q, k_cache, v_cache, proxy_keys, q_idx, idx_w, out, idx_out, d);
  if (s) return s;
  if (!ws || ws_bytes < d.total)
    return fail(TKA_ERR_WORKSPACE, "decode needs %zu workspace bytes (got %zu)", d.total, ws_bytes);
  if (!aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  return run_decode(p, q, k_cache, v_cache, proxy_keys, q_idx, idx_w, out, idx_out, d, static_cast<char*>(ws),
                    as_stream(stream));
}

// ---- the fused step without a workspace argument ----
// Scratch of topk_decode_noalloc: a file-scope device array. In host code its
// name is only a stand-in: its device address, one per GPU, comes from
// hipGetSymbolAddress on the first call on that device, and only that address
// is handed to kernels.
static __device__ __align__(256) uint8_t scratch[TKA_NOALLOC_SCRATCH_BYTES];

}  // extern "C"

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of the scratch array (looked up once per device)
tka_status scratch_for_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    const hipError_t e = hipGetLastError();
    return fail(TKA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(TKA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev,
                                                 kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(TKA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return TKA_OK;
}
}  // namespace

extern "C" {

tka_status topk_decode_noalloc(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                               const void* proxy_keys, const void* q_idx, const float* idx_w, float* out,
                               int32_t* idx_out, void* stream) {
  DecodeLayout d;
  tka_status s = check_decode_call(p, q, k_cache, v_cache, proxy_keys, q_idx, idx_w, out, idx_out, d);
  if (s) return s;
  if (d.total > (size_t)TKA_NOALLOC_SCRATCH_BYTES)
    return fail(TKA_ERR_UNSUPPORTED, "this step needs %zu scratch bytes, more than the %zu of topk_decode_noalloc",
                d.total, (size_t)TKA_NOALLOC_SCRATCH_BYTES);
  char* base = nullptr;
  if ((s = scratch_for_current_device(&base))) return s;
  return run_decode(p, q, k_cache, v_cache, proxy_keys, q_idx, idx_w, out, idx_out, d, base, as_stream(stream));
}

// ---- certified adaptive step: full exact scores -> adaptive k -> gather ----
}  // extern "C"

namespace {
struct AdaptiveLayout {
  size_t scores, idx, selv, kout, tau, scratch, gather_ws, rmax, total;
  int64_t rows;
  int rslots;  // partial row maxima written by the scoring pass (0: none)
  GatherPlan gp;
};
AdaptiveLayout adaptive_layout(const tka_problem* p) {
  AdaptiveLayout d;
  d.rows = score_rows(p);
  const int32_t len = score_len(p);
  size_t o = 0;
  d.scores = o;
  o += al256(sizeof(float) * (size_t)d.rows * (len > 0 ? len : 1));
  d.idx = o;
  o += al256(sizeof(int32_t) * (size_t)d.rows * p->top_k);
  d.selv = o;
  o += al256(sizeof(float) * (size_t)d.rows * p->top_k);
  d.kout = o;
  o += al256(sizeof(int32_t) * (size_t)d.rows);
  d.tau = o;
  o += al256(sizeof(float) * (size_t)d.rows);
  d.scratch = o;
  o += adaptive_scratch(d.rows).total;
  d.gather_ws = o;
  GatherArgs ga = gather_args(p, nullptr, nullptr, nullptr, nullptr, p->top_k, 0, 0, nullptr, nullptr);
  d.gp = plan_gather(ga);
  o += al256(d.gp.ws_bytes);
  d.rmax = o;
  d.rslots = score_rmax_slots(dense_score_args(p, nullptr, nullptr, nullptr));
  o += al256(sizeof(uint32_t) * (size_t)d.rows * (size_t)d.rslots);
  d.total = o;
  return d;
}
tka_status check_adaptive_problem(const tka_problem* p) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (nqry(p) > 1) return fail(TKA_ERR_UNSUPPORTED, "the certified step takes one query per sequence");
  if (p->mode != TKA_SCORE_EXACT) return fail(TKA_ERR_INVALID_ARG, "the adaptive step needs TKA_SCORE_EXACT");
  return check_gather_shape(p, p->top_k, 0, 0, nullptr);
}
}  // namespace

extern "C" {

tka_status topk_decode_adaptive_workspace_size(const tka_problem* p, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  tka_status s = check_adaptive_problem(p);
  if (s) return s;
  *bytes = adaptive_layout(p).total;
  return ok();
}

tka_status topk_decode_adaptive(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                float eps, int32_t k_min, float* out, int32_t* idx_out, int32_t* k_out,
                                float* tau_out, void* ws, size_t ws_bytes, void* stream) {
  tka_status s = check_adaptive_problem(p);
  if (s) return s;
  if ((s = check_attn_ptrs(p, q, k_cache, v_cache, out))) return s;
  const AdaptiveLayout d = adaptive_layout(p);
  const Range o = span_of(out, out_bytes(p));
  const Range kv = span_of(k_cache, kv_bytes(p)), vv = span_of(v_cache, kv_bytes(p)), qq = span_of(q, attn_q_bytes(p));
  Range io{};
  if (idx_out) {
    if (reinterpret_cast<uintptr_t>(idx_out) & 3) return fail(TKA_ERR_ALIGNMENT, "idx_out is not 4-byte aligned");
    io = span_of(idx_out, sizeof(int32_t) * (size_t)d.rows * p->top_k);
    if (overlap(io, o) || overlap(io, kv) || overlap(io, vv) || overlap(io, qq))
      return fail(TKA_ERR_INVALID_ARG, "idx_out overlaps another buffer");
  }
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(TKA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (k_min < 0) return fail(TKA_ERR_INVALID_ARG, "k_min must be >= 0");
  for (const void* ptr : {(const void*)k_out, (const void*)tau_out}) {
    if (!ptr) continue;
    if (reinterpret_cast<uintptr_t>(ptr) & 3) return fail(TKA_ERR_ALIGNMENT, "k_out / tau_out not 4-byte aligned");
    const Range r = span_of(ptr, sizeof(int32_t) * (size_t)d.rows);
    if (overlap(r, o) || overlap(r, kv) || overlap(r, vv) || overlap(r, qq) || (idx_out && overlap(r, io)))
      return fail(TKA_ERR_INVALID_ARG, "k_out or tau_out overlaps another buffer");
  }
  if (k_out && tau_out && overlap(span_of(k_out, 4 * (size_t)d.rows), span_of(tau_out, 4 * (size_t)d.rows)))
    return fail(TKA_ERR_INVALID_ARG, "k_out overlaps tau_out");
  if (!ws || ws_bytes < d.total)
    return fail(TKA_ERR_WORKSPACE, "adaptive decode needs %zu workspace bytes (got %zu)", d.total, ws_bytes);
  if (!aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + d.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + d.idx);
  float* selv = reinterpret_cast<float*>(base + d.selv);
  int32_t* kk = k_out ? k_out : reinterpret_cast<int32_t*>(base + d.kout);
  float* tau = tau_out ? tau_out : reinterpret_cast<float*>(base + d.tau);
  const AdaptiveScratch sc = adaptive_scratch(d.rows);
  const int32_t len = score_len(p);
  // the scores, with each row's partial maxima beside them where the scoring kernel writes them
  uint32_t* rmax = d.rslots > 0 ? reinterpret_cast<uint32_t*>(base + d.rmax) : nullptr;
  ScoreArgs sa_score = dense_score_args(p, q, k_cache, scores);
  sa_score.rmax = rmax;
  launch_score_dense(sa_score, st);
  SelectArgs sa{scores, d.rows, len, (int64_t)len, p->top_k, idx, selv};
  launch_select_adaptive(sa, eps, k_min, kk, reinterpret_cast<uint64_t*>(base + d.scratch + sc.W),
                         reinterpret_cast<float*>(base + d.scratch + sc.M),
                         reinterpret_cast<uint32_t*>(base + d.scratch + sc.flag), tau, st, rmax, d.rslots);
  GatherArgs ga = gather_args(p, q, k_cache, v_cache, idx, p->top_k, 0, 0, selv, out);
  launch_gather(ga, d.gp, base + d.gather_ws, st);
  return launched("topk_decode_adaptive");
}

// ---- two-level step ----
}  // extern "C"

namespace {
struct HisaLayout {
  size_t bscores, blk, sel_ws, cand, krow, idx, selv, gather_ws, total;
  int64_t rows, m, ncand;
  GatherPlan gp;
};
HisaLayout hisa_layout(const tka_problem* p) {
  HisaLayout d;
  d.rows = (int64_t)p->batch * p->n_q_heads;
  d.m = n_blocks(p);
  d.ncand = (int64_t)p->top_blocks * p->block_size;
  size_t o = 0;
  d.bscores = o;
  o += al256(sizeof(float) * (size_t)(d.rows * d.m));
  d.blk = o;
  o += al256(sizeof(int32_t) * (size_t)(d.rows * p->top_blocks));
  d.sel_ws = o;
  o += al256(select_workspace_bytes(d.rows, (int)d.m, p->top_blocks));
  d.cand = o;
  o += al256(sizeof(float) * (size_t)(d.rows * d.ncand));
  d.krow = o;
  o += al256(sizeof(int32_t) * (size_t)d.rows);
  d.idx = o;
  o += al256(sizeof(int32_t) * (size_t)(d.rows * p->top_k));
  d.selv = o;
  o += al256(sizeof(float) * (size_t)(d.rows * p->top_k));
  d.gather_ws = o;
  GatherArgs ga = gather_args(p, nullptr, nullptr, nullptr, nullptr, p->top_k, 0, 0, nullptr, nullptr);
  d.gp = plan_gather(ga);
  o += al256(d.gp.ws_bytes);
  d.total = o;
  return d;
}
tka_status check_hisa_problem(const tka_problem* p) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (p->mode != TKA_SCORE_HISA) return fail(TKA_ERR_INVALID_ARG, "topk_hisa_decode needs mode TKA_SCORE_HISA");
  if ((int64_t)p->top_blocks * p->block_size > 0x7fffffff / 4)
    return fail(TKA_ERR_UNSUPPORTED, "top_blocks * block_size too large");
  if (!select_len_supported(score_rows(p), score_len(p)))
    return fail(TKA_ERR_UNSUPPORTED, "too many blocks for %lld rows (at most about 12M)", (long long)score_rows(p));
  return check_gather_shape(p, p->top_k, 0, 0, nullptr);
}
}  // namespace

extern "C" {

tka_status topk_hisa_decode_workspace_size(const tka_problem* p, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  tka_status s = check_hisa_problem(p);
  if (s) return s;
  *bytes = hisa_layout(p).total;
  return ok();
}

tka_status topk_hisa_decode(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                            const float* means, float* out, int32_t* idx_out, int32_t* blk_out,
                            float* block_scores_out, float* cand_scores_out, void* ws, size_t ws_bytes,
                            void* stream) {
  tka_status s = check_hisa_problem(p);
  if (s) return s;
  if ((s = check_attn_ptrs(p, q, k_cache, v_cache, out))) return s;
  if ((s = need_ptr(means, "means"))) return s;
  const HisaLayout d = hisa_layout(p);
  const Range o = span_of(out, out_bytes(p)), mo = span_of(means, proxy_bytes(p));
  const Range kv = span_of(k_cache, kv_bytes(p)), vv = span_of(v_cache, kv_bytes(p)), qq = span_of(q, attn_q_bytes(p));
  if (overlap(o, mo)) return fail(TKA_ERR_INVALID_ARG, "out overlaps means");
  struct Opt {
    const void* ptr;
    size_t bytes;
    const char* name;
  } opts[4] = {{idx_out, sizeof(int32_t) * (size_t)(d.rows * p->top_k), "idx_out"},
               {blk_out, sizeof(int32_t) * (size_t)(d.rows * p->top_blocks), "blk_out"},
               {block_scores_out, sizeof(float) * (size_t)(d.rows * d.m), "block_scores_out"},
               {cand_scores_out, sizeof(float) * (size_t)(d.rows * d.ncand), "cand_scores_out"}};
  for (int i = 0; i < 4; ++i) {
    if (!opts[i].ptr) continue;
    if (reinterpret_cast<uintptr_t>(opts[i].ptr) & 3) return fail(TKA_ERR_ALIGNMENT, "%s not 4-byte aligned", opts[i].name);
    const Range r = span_of(opts[i].ptr, opts[i].bytes);
    if (overlap(r, o) || overlap(r, mo) || overlap(r, kv) || overlap(r, vv) || overlap(r, qq))
      return fail(TKA_ERR_INVALID_ARG, "%s overlaps an input or out", opts[i].name);
    for (int j = 0; j < i; ++j)
      if (opts[j].ptr && overlap(r, span_of(opts[j].ptr, opts[j].bytes)))
        return fail(TKA_ERR_INVALID_ARG, "%s overlaps %s", opts[i].name, opts[j].name);
  }
  if (!ws || ws_bytes < d.total)
    return fail(TKA_ERR_WORKSPACE, "two-level decode needs %zu workspace bytes (got %zu)", d.total, ws_bytes);
  if (!aligned16(ws)) return fail(TKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

  hipStream_t st = as_stream(stream);
  char* base = static_cast<char*>(ws);
  float* bscores = block_scores_out ? block_scores_out : reinterpret_cast<float*>(base + d.bscores);
  int32_t* blk = blk_out ? blk_out : reinterpret_cast<int32_t*>(base + d.blk);
  float* cand = cand_scores_out ? cand_scores_out : reinterpret_cast<float*>(base + d.cand);
  int32_t* krow = reinterpret_cast<int32_t*>(base + d.krow);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + d.idx);
  float* selv = reinterpret_cast<float*>(base + d.selv);
  // coarse level: every block's score from the means, the top K_B blocks
  run_score(p, q, means, nullptr, bscores, st);
  SelectArgs sb{bscores, d.rows, (int)d.m, d.m, p->top_blocks, blk, nullptr};
  launch_select(sb, base + d.sel_ws, st);
  // fine level: exact scores of the kept blocks' tokens, the top k' of them
  HisaArgs ha;
  ha.q = q;
  ha.K = k_cache;
  ha.blk = blk;
  ha.cand = cand;
  ha.krow = krow;
  ha.B = p->batch;
  ha.Hq = p->n_q_heads;
  ha.G = p->n_q_heads / p->n_kv_heads;
  ha.d = p->head_dim;
  ha.L = p->seq_len;
  ha.KB = p->top_blocks;
  ha.bsz = p->block_size;
  ha.k = p->top_k;
  ha.sb = p->kv_stride_b;
  ha.sh = p->kv_stride_h;
  ha.sl = p->kv_stride_l;
  ha.scale = eff_scale(p);
  ha.bf16 = p->qkv_dtype == TKA_BF16;
  launch_hisa_token_scores(ha, st);
  SelectArgs sc{cand, d.rows, (int)d.ncand, d.ncand, p->top_k, idx, selv};
  launch_select_rows_counts(sc, krow, st);
  launch_hisa_map(idx, blk, d.rows, p->top_k, p->top_blocks, p->block_size, st);
  // attention over the kept tokens, their exact scores as logits
  GatherArgs ga = gather_args(p, q, k_cache, v_cache, idx, p->top_k, 0, 0, selv, out);
  launch_gather(ga, d.gp, base + d.gather_ws, st);
  return launched("topk_hisa_decode");
}

tka_status topk_workspace_size(const tka_problem* p, int32_t which, size_t* bytes) {
  if (!bytes) return fail(TKA_ERR_INVALID_ARG, "bytes is NULL");
  tka_status s = check_attn_shape(p);
  if (s) return s;
  switch (which) {
    case TKA_WS_SELECT: {
      const int64_t rows = p->mode == TKA_SCORE_HISA ? (int64_t)p->batch * p->n_q_heads : score_rows(p);
      *bytes = select_workspace_bytes(rows, score_len(p), p->top_k);
      return ok();
    }
    case TKA_WS_GATHER:
      return sparse_attn_gather_workspace_size(p, p->top_k, p->mode == TKA_SCORE_BLOCK_MEAN ? p->block_size : 0,
                                               p->mode == TKA_SCORE_INDEXER ? 1 : 0, bytes);
    case TKA_WS_DECODE:
      return p->mode == TKA_SCORE_HISA ? topk_hisa_decode_workspace_size(p, bytes)
                                       : topk_decode_workspace_size(p, bytes);
    case TKA_WS_DECODE_ADAPTIVE:
      return topk_decode_adaptive_workspace_size(p, bytes);
    default:
      return fail(TKA_ERR_INVALID_ARG, "unknown workspace kind %d", which);
  }
}

tka_status topk_block_mean_build(const tka_problem* p, const void* k_cache, float* means, void* stream) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (p->mode != TKA_SCORE_BLOCK_MEAN && p->mode != TKA_SCORE_HISA)
    return fail(TKA_ERR_INVALID_ARG, "mode must be TKA_SCORE_BLOCK_MEAN or TKA_SCORE_HISA");
  if ((s = need_ptr(k_cache, "k_cache")) || (s = need_ptr(means, "means"))) return s;
  const Range mo = span_of(means, proxy_bytes(p));
  if (overlap(mo, span_of(k_cache, kv_bytes(p)))) return fail(TKA_ERR_INVALID_ARG, "means overlaps k_cache");
  BlockMeanArgs a;
  a.K = k_cache;
  a.means = means;
  a.B = p->batch;
  a.Hkv = p->n_kv_heads;
  a.d = p->head_dim;
  a.L = p->seq_len;
  a.bsz = p->block_size;
  a.m = (int)mean_slots(p);
  a.sb = p->kv_stride_b;
  a.sh = p->kv_stride_h;
  a.sl = p->kv_stride_l;
  a.bf16 = p->qkv_dtype == TKA_BF16;
  a.j0 = 0;
  a.j1 = (int)n_blocks(p);
  launch_block_mean(a, as_stream(stream));
  return launched("topk_block_mean_build");
}

tka_status topk_cache_append(const tka_problem* p, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const float* kI_new, void* kI_cache, float* means, void* stream) {
  tka_status s = check_attn_shape(p);
  if (s) return s;
  if (nqry(p) > 1) return fail(TKA_ERR_UNSUPPORTED, "append one position at a time (n_queries 0 or 1)");
  const bool kv = k_new || v_new;
  if (kv) {
    if ((s = need_ptr(k_new, "k_new")) || (s = need_ptr(v_new, "v_new")) || (s = need_ptr(k_cache, "k_cache")) ||
        (s = need_ptr(v_cache, "v_cache")))
      return s;
  }
  if (means) {
    if (p->mode != TKA_SCORE_BLOCK_MEAN && p->mode != TKA_SCORE_HISA)
      return fail(TKA_ERR_INVALID_ARG, "means only with TKA_SCORE_BLOCK_MEAN or TKA_SCORE_HISA");
    if ((s = need_ptr(means, "means")) || (s = need_ptr(k_cache, "k_cache"))) return s;
  }
  if (kI_new || kI_cache) {
    if (p->mode != TKA_SCORE_INDEXER) return fail(TKA_ERR_INVALID_ARG, "kI_new/kI_cache only with TKA_SCORE_INDEXER");
    if ((s = need_ptr(kI_new, "kI_new", false)) || (s = need_ptr(kI_cache, "kI_cache", false))) return s;
    if (reinterpret_cast<uintptr_t>(kI_new) & 3) return fail(TKA_ERR_ALIGNMENT, "kI_new is not 4-byte aligned");
  }
  const size_t row_bytes = (size_t)p->head_dim * esize(p->qkv_dtype);
  const size_t new_bytes = row_bytes * (size_t)p->batch * p->n_kv_heads;
  const Range kc = k_cache ? span_of(k_cache, kv_bytes(p)) : Range{}, vc = v_cache ? span_of(v_cache, kv_bytes(p)) : Range{};
  if (kv) {
    const Range kn = span_of(k_new, new_bytes), vn = span_of(v_new, new_bytes);
    if (overlap(kc, vc) || overlap(kn, kc) || overlap(kn, vc) || overlap(vn, kc) || overlap(vn, vc))
      return fail(TKA_ERR_INVALID_ARG, "the new rows or the caches overlap");
  }
  if (means) {
    const Range mo = span_of(means, proxy_bytes(p));
    if (overlap(mo, kc) || overlap(mo, vc)) return fail(TKA_ERR_INVALID_ARG, "means overlaps a cache");
  }
  if (kI_cache) {
    const Range ko = span_of(kI_cache, proxy_bytes(p));
    if (overlap(ko, span_of(kI_new, sizeof(float) * (size_t)p->batch * p->idx_dim)) || overlap(ko, kc) ||
        overlap(ko, vc))
      return fail(TKA_ERR_INVALID_ARG, "kI_cache overlaps another buffer");
  }
  hipStream_t st = as_stream(stream);
  const int pos = p->seq_len - 1;
  if (kv)
    launch_append_rows(k_new, v_new, k_cache, v_cache, p->batch, p->n_kv_heads, (int)row_bytes,
                       (int)esize(p->qkv_dtype), p->kv_stride_b, p->kv_stride_h, p->kv_stride_l, pos, st);
  if (means) {  // the block holding pos, recomputed from the cache as topk_block_mean_build does
    BlockMeanArgs a;
    a.K = k_cache;
    a.means = means;
    a.B = p->batch;
    a.Hkv = p->n_kv_heads;
    a.d = p->head_dim;
    a.L = p->seq_len;
    a.bsz = p->block_size;
    a.m = (int)mean_slots(p);
    a.sb = p->kv_stride_b;
    a.sh = p->kv_stride_h;
    a.sl = p->kv_stride_l;
    a.bf16 = p->qkv_dtype == TKA_BF16;
    a.j0 = pos / p->block_size;
    a.j1 = a.j0 + 1;
    launch_block_mean(a, st);
  }
  if (kI_cache)
    launch_append_indexer(kI_new, static_cast<uint8_t*>(kI_cache), p->batch, p->idx_dim, (int)idx_slots(p), pos, st);
  return launched("topk_cache_append");
}

}  // extern "C"
