/*
 * oracle.c - plain, slow fp64 CPU oracle for one top-k sparse attention
 * decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library. The GPU library neither includes
 * nor links it, and it includes nothing of the GPU library.
 *
 * What it computes, in the order the pages give it ("Sparse Attention in LLM
 * Inference: Practical Trade-Offs", "The Role of the Indexer": score every
 * earlier position for the current query, keep the Top-K, attend only over
 * those; the same two steps in "Evolution of Sparse Attention in Long-Context
 * LLMs", section 2):
 *   1. score   - exact token score s_i = f(q_t, k_i) ("Sparse Attention
 *                Landscape", "Token Sparse Attention"), here scale * <q, k_i>;
 *                block score s_j = f(q_t, B_j) with f = <q, mean of the keys
 *                of block j> (same page, "Block Sparse Attention", MoBA);
 *                indexer score sum_j w_j ReLU(<q^I_j, k^I_i>) (same page,
 *                "Token Sparse Attention", lightning indexer).
 *   2. select  - TopK over the scores (same page, "Block Sparse Attention",
 *                the TopK_j s_j formula). Ties at the k-th score go to the
 *                lower position; NaN ranks below every number; -0 equals +0.
 *                The kept positions are emitted ascending, padded with -1.
 *   3. attend  - exact softmax attention over the kept keys and values only
 *                (dense attention Attention(Q_t, K_1:t, V_1:t) of "Sparse
 *                Attention in LLM Inference", "The Bottleneck of Dense
 *                Attention", restricted to the kept set).
 * Every input is decoded exactly to double (fp32, bf16 by bit shift, OCP
 * E4M3FN by its definition) and all arithmetic is fp64. Sorting uses the C
 * library's qsort with the total order above as comparator.
 *
 * Diagnostics (exact variant) follow "A Mathematical Theory of Top-k Sparse
 * Attention via Total Variation Distance" (abstract): the full softmax P, the
 * truncated and renormalised P-hat, the discarded tail mass tau, TV(P,P-hat),
 * KL(P-hat||P), the head/tail means of V and the entropy of P.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_E4M3 = 2 };
enum { OMODE_EXACT = 0, OMODE_BLOCK = 1, OMODE_INDEXER = 2 };

typedef struct {
  int32_t B, Hq, Hkv, d, L, k;
  int64_t sb, sh, sl; /* K/V element strides of batch, kv head, position; dims contiguous */
  int32_t dt;         /* dtype of q, K, V */
  double scale;       /* attention logit scale; <= 0 means 1/sqrt(d) */
  int32_t mode;
  int32_t block; /* block size b (block variant) */
  int32_t HI, dI; /* indexer heads and dim (indexer variant, E4M3FN) */
} orc_problem;

/* ---- exact decoding of stored numbers ---- */

double orc_dec_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN. */
double orc_dec_e4m3(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

/* Encoding to OCP E4M3FN for keys stored in the indexer cache (the appended
 * low-dimensional key of "Sparse Attention Landscape", "Token Sparse
 * Attention"): the finite code nearest to |x|, a tie going to the code with an
 * even mantissa; |x| >= 448 (the largest finite value, infinities included)
 * saturates to 448; NaN encodes as 0x7f; the sign bit is kept (also for 0).
 * Found by looking at every code: plain and slow on purpose. */
static uint8_t enc_e4m3(double x) {
  if (isnan(x)) return 0x7f;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs(x);
  if (a >= 448.0) return sign | 0x7e;
  int best = 0;
  double dbest = a;
  for (int c = 1; c <= 0x7e; ++c) {
    const double dc = fabs(orc_dec_e4m3((uint8_t)c) - a);
    if (dc < dbest || (dc == dbest && (c & 1) == 0)) {
      best = c;
      dbest = dc;
    }
  }
  return sign | (uint8_t)best;
}

void orc_encode_e4m3(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = enc_e4m3((double)x[i]);
}

static double ld(const void* p, int dt, int64_t i) {
  if (dt == ODT_F32) return (double)((const float*)p)[i];
  if (dt == ODT_BF16) return orc_dec_bf16(((const uint16_t*)p)[i]);
  return orc_dec_e4m3(((const uint8_t*)p)[i]);
}

void orc_decode_buf(int dt, const void* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = ld(src, dt, i);
}

static double attn_scale(const orc_problem* p) { return p->scale > 0 ? p->scale : 1.0 / sqrt((double)p->d); }

static int64_t n_blocks(const orc_problem* p) { return (p->L + p->block - 1) / p->block; }

static int64_t score_row_len(const orc_problem* p) {
  if (p->mode == OMODE_BLOCK) return n_blocks(p) - 1; /* the current block does not compete */
  return p->L;
}

static int64_t kv_off(const orc_problem* p, int64_t b, int64_t g, int64_t i) {
  return b * p->sb + g * p->sh + i * p->sl;
}

/* <q[b,h], K[b,g(h),i]> in fp64 */
static double qk(const orc_problem* p, const void* q, const void* K, int64_t b, int64_t h, int64_t i) {
  const int64_t G = p->Hq / p->Hkv, g = h / G;
  const int64_t qo = (b * p->Hq + h) * p->d, ko = kv_off(p, b, g, i);
  double s = 0;
  for (int64_t c = 0; c < p->d; ++c) s += ld(q, p->dt, qo + c) * ld(K, p->dt, ko + c);
  return s;
}

/*
 * Step 1: scores for the rows listed in `rows` (NULL = all rows).
 *  exact:   row r = b*Hq + h, length L:      scale * <q[b,h], K[b,g,i]>
 *  block:   row r = b*Hq + h, length m - 1:  <q[b,h], mean_{i in B_j} K[b,g,i]>, no scale
 *           (B_j = [j b, min((j+1) b, L)); the current block m-1 is left out)
 *  indexer: row r = b, length L:             sum_j w[b,j] * max(0, <qI[b,j], kI[b,i]>), no scale
 */
int orc_score(const orc_problem* p, const void* q, const void* K, const void* qI, const void* kI, const float* w,
              const int64_t* rows, int64_t n_rows, double* out) {
  const int64_t len = score_row_len(p);
  const double sc = attn_scale(p);
  if (p->mode == OMODE_INDEXER) {
    for (int64_t r = 0; r < n_rows; ++r) {
      const int64_t b = rows ? rows[r] : r;
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < p->L; ++i) {
        double acc = 0;
        for (int64_t j = 0; j < p->HI; ++j) {
          double dot = 0;
          for (int64_t c = 0; c < p->dI; ++c)
            dot += ld(qI, ODT_E4M3, (b * p->HI + j) * p->dI + c) * ld(kI, ODT_E4M3, (b * p->L + i) * p->dI + c);
          acc += (double)w[b * p->HI + j] * (dot > 0 ? dot : 0.0);
        }
        out[r * len + i] = acc;
      }
    }
    return 0;
  }
  const int64_t G = p->Hq / p->Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int64_t b = row / p->Hq, h = row % p->Hq, g = h / G;
    if (p->mode == OMODE_EXACT) {
      for (int64_t i = 0; i < p->L; ++i) out[r * len + i] = sc * qk(p, q, K, b, h, i);
    } else {
      double* mu = (double*)malloc(sizeof(double) * (size_t)p->d);
      for (int64_t j = 0; j < len; ++j) {
        const int64_t i0 = j * p->block, i1 = (i0 + p->block < p->L) ? i0 + p->block : p->L;
        for (int64_t c = 0; c < p->d; ++c) mu[c] = 0;
        for (int64_t i = i0; i < i1; ++i)
          for (int64_t c = 0; c < p->d; ++c) mu[c] += ld(K, p->dt, kv_off(p, b, g, i) + c);
        double s = 0;
        for (int64_t c = 0; c < p->d; ++c) s += ld(q, p->dt, (b * p->Hq + h) * p->d + c) * (mu[c] / (double)(i1 - i0));
        out[r * len + j] = s;
      }
      free(mu);
    }
  }
  return 0;
}

/* Block-mean keys of the block variant, all m = ceil(L/b) blocks (the partial
 * last one over its own keys): means[b,g,j,c] = (1/n_j) sum over block j of
 * K[b,g,i,c] ("Sparse Attention Landscape", "Block Sparse Attention": MoBA
 * mean-pools the keys of each block). fp64, [B,Hkv,m,d] contiguous. */
int orc_block_means(const orc_problem* p, const void* K, double* means) {
  const int64_t m = n_blocks(p);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < p->B; ++b)
    for (int64_t g = 0; g < p->Hkv; ++g)
      for (int64_t j = 0; j < m; ++j) {
        const int64_t i0 = j * p->block, i1 = (i0 + p->block < p->L) ? i0 + p->block : p->L;
        double* mu = means + ((b * p->Hkv + g) * m + j) * p->d;
        for (int64_t c = 0; c < p->d; ++c) mu[c] = 0;
        for (int64_t i = i0; i < i1; ++i)
          for (int64_t c = 0; c < p->d; ++c) mu[c] += ld(K, p->dt, kv_off(p, b, g, i) + c);
        for (int64_t c = 0; c < p->d; ++c) mu[c] /= (double)(i1 - i0);
      }
  return 0;
}

/* ---- step 2: exact top-k under the total order ---- */

typedef struct {
  double v;
  int64_t i;
} vi_t;

/* a before b  <=>  v_a > v_b, or v_a == v_b and i_a < i_b; NaN after every number */
static int cmp_rank(const void* a, const void* b) {
  const vi_t *x = (const vi_t*)a, *y = (const vi_t*)b;
  const int xn = isnan(x->v), yn = isnan(y->v);
  if (xn != yn) return xn ? 1 : -1;
  if (!xn && x->v != y->v) return x->v > y->v ? -1 : 1;
  return (x->i > y->i) - (x->i < y->i);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static void select_row(vi_t* tmp, int64_t len, int64_t k, int32_t* idx) {
  qsort(tmp, (size_t)len, sizeof(vi_t), cmp_rank);
  const int64_t kk = k < len ? k : len;
  for (int64_t j = 0; j < kk; ++j) idx[j] = (int32_t)tmp[j].i;
  qsort(idx, (size_t)kk, sizeof(int32_t), cmp_i32);
  for (int64_t j = kk; j < k; ++j) idx[j] = -1;
}

int orc_select_f64(const double* s, int64_t n_rows, int64_t len, int64_t stride, int64_t k, int32_t* idx) {
  if (k <= 0 || len < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)(len > 0 ? len : 1));
    for (int64_t i = 0; i < len; ++i) {
      tmp[i].v = s[r * stride + i];
      tmp[i].i = i;
    }
    select_row(tmp, len, k, idx + r * k);
    free(tmp);
  }
  return 0;
}

/* the same order on a float array (fp32 values are exact in double) */
int orc_select_f32(const float* s, int64_t n_rows, int64_t len, int64_t stride, int64_t k, int32_t* idx) {
  if (k <= 0 || len < 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)(len > 0 ? len : 1));
    for (int64_t i = 0; i < len; ++i) {
      tmp[i].v = (double)s[r * stride + i];
      tmp[i].i = i;
    }
    select_row(tmp, len, k, idx + r * k);
    free(tmp);
  }
  return 0;
}

/* ---- step 2, certified variant: the smallest k meeting a total-variation budget ----
 * "A Mathematical Theory of Top-k Sparse Attention via Total Variation Distance"
 * (abstract): the TV distance between the softmax P of a row and its top-k
 * truncation equals the softmax mass the truncation discards, so the smallest k
 * with TV <= eps is the smallest k whose top-k (in the select order) holds at
 * least 1 - eps of the mass. Masses are exp(s_i - max s) in fp64 (NaN: no mass;
 * an element equal to the maximum has mass 1, also when the maximum is +inf),
 * the discarded mass of the first k is the sum of the masses after them, added
 * from the smallest up. k is then clamped to [max(k_min, 1), min(k_max, len)];
 * tau = discarded mass / total for the final k (NaN when no element has mass).
 * Kept positions ascending, then -1 up to k_max. */
static void adaptive_row(vi_t* tmp, int64_t len, double eps, int64_t k_min, int64_t k_max, int32_t* idx,
                         int32_t* k_out, double* tau_out) {
  qsort(tmp, (size_t)len, sizeof(vi_t), cmp_rank);
  double* tail = (double*)malloc(sizeof(double) * (size_t)(len + 1));
  const double M = (len > 0 && !isnan(tmp[0].v)) ? tmp[0].v : NAN;
  tail[len] = 0.0;
  for (int64_t j = len - 1; j >= 0; --j) {
    const double v = tmp[j].v;
    const double w = isnan(v) || isnan(M) ? 0.0 : (v == M ? 1.0 : exp(v - M));
    tail[j] = tail[j + 1] + w;
  }
  const double Z = tail[0];
  int64_t k = len;
  for (int64_t j = 0; j <= len; ++j)  /* a row without mass needs no key: k = 0 before the clamp */
    if (tail[j] <= eps * Z) {
      k = j;
      break;
    }
  int64_t lo = k_min > 1 ? k_min : 1, hi = k_max < len ? k_max : len;
  if (k < lo) k = lo;
  if (k > hi) k = hi;
  *k_out = (int32_t)k;
  *tau_out = Z > 0.0 ? tail[k] / Z : NAN;
  for (int64_t j = 0; j < k; ++j) idx[j] = (int32_t)tmp[j].i;
  qsort(idx, (size_t)k, sizeof(int32_t), cmp_i32);
  for (int64_t j = k; j < k_max; ++j) idx[j] = -1;
  free(tail);
}

/* fp32 logits (exact in double), rows of len at the given stride */
int orc_select_adaptive_f32(const float* s, int64_t n_rows, int64_t len, int64_t stride, double eps, int64_t k_min,
                            int64_t k_max, int32_t* idx, int32_t* k_out, double* tau_out) {
  if (k_max <= 0 || len < 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)(len > 0 ? len : 1));
    for (int64_t i = 0; i < len; ++i) {
      tmp[i].v = (double)s[r * stride + i];
      tmp[i].i = i;
    }
    adaptive_row(tmp, len, eps, k_min, k_max, idx + r * k_max, k_out + r, tau_out + r);
    free(tmp);
  }
  return 0;
}

int orc_select_adaptive_f64(const double* s, int64_t n_rows, int64_t len, int64_t stride, double eps, int64_t k_min,
                            int64_t k_max, int32_t* idx, int32_t* k_out, double* tau_out) {
  if (k_max <= 0 || len < 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)(len > 0 ? len : 1));
    for (int64_t i = 0; i < len; ++i) {
      tmp[i].v = s[r * stride + i];
      tmp[i].i = i;
    }
    adaptive_row(tmp, len, eps, k_min, k_max, idx + r * k_max, k_out + r, tau_out + r);
    free(tmp);
  }
  return 0;
}

/* ---- step 3: exact softmax attention over a kept set ---- */

/* token list of one row: unit 0 = positions; unit b >= 1 = block ids of b keys, plus the current block */
static int64_t expand(const orc_problem* p, const int32_t* list, int64_t n, int64_t unit, int64_t* tok) {
  int64_t t = 0;
  if (unit <= 0) {
    for (int64_t j = 0; j < n; ++j)
      if (list[j] >= 0 && list[j] < p->L) tok[t++] = list[j];
    return t;
  }
  const int64_t m = (p->L + unit - 1) / unit;
  for (int64_t j = 0; j < n; ++j) {
    if (list[j] < 0 || list[j] >= m - 1) continue;
    for (int64_t i = list[j] * unit; i < (list[j] + 1) * unit && i < p->L; ++i) tok[t++] = i;
  }
  for (int64_t i = (m - 1) * unit; i < p->L; ++i) tok[t++] = i;
  return t;
}

/*
 * rows: b*Hq + h (NULL = all). out [n_rows, d]. Where the kept list of a row is:
 *   list_mode 0: idx[(b*Hq + h) * n_idx]   (one set per query head)
 *   list_mode 1: idx[b * n_idx]            (one set per sequence, shared by its heads)
 *   list_mode 2: idx[r * n_idx]            (r = position of the row in `rows`)
 *   list_mode 3: idx[0]                    (one set for every row)
 */
int orc_attend(const orc_problem* p, const void* q, const void* K, const void* V, const int32_t* idx, int64_t n_idx,
               int64_t unit, int32_t list_mode, const int64_t* rows, int64_t n_rows, double* out) {
  const int64_t G = p->Hq / p->Hkv;
  const double sc = attn_scale(p);
  const int64_t cap = (unit <= 0) ? n_idx : n_idx * unit + unit;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int64_t b = row / p->Hq, h = row % p->Hq, g = h / G;
    const int64_t li = list_mode == 0 ? row : list_mode == 1 ? b : list_mode == 2 ? r : 0;
    const int32_t* list = idx + li * n_idx;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    const int64_t nt = expand(p, list, n_idx, unit, tok);
    double* o = out + r * p->d;
    for (int64_t c = 0; c < p->d; ++c) o[c] = 0;
    if (nt == 0) {
      bad |= 1;
    } else {
      double M = -INFINITY;
      for (int64_t t = 0; t < nt; ++t) {
        z[t] = sc * qk(p, q, K, b, h, tok[t]);
        if (z[t] > M) M = z[t];
      }
      double Z = 0;
      for (int64_t t = 0; t < nt; ++t) {
        const double wt = exp(z[t] - M);
        Z += wt;
        const int64_t vo = kv_off(p, b, g, tok[t]);
        for (int64_t c = 0; c < p->d; ++c) o[c] += wt * ld(V, p->dt, vo + c);
      }
      for (int64_t c = 0; c < p->d; ++c) o[c] /= Z;
    }
    free(tok);
    free(z);
  }
  return bad ? 1 : 0;
}

/*
 * Whole step: score -> select -> attend.
 * exact / block: rows are b*Hq + h; idx_out [n_rows, k]; out [n_rows, d].
 * indexer:       rows are b; idx_out [n_rows, k] (shared); out [n_rows, Hq, d].
 */
int orc_decode(const orc_problem* p, const void* q, const void* K, const void* V, const void* qI, const void* kI,
               const float* w, const int64_t* rows, int64_t n_rows, double* out, int32_t* idx_out) {
  const int64_t len = score_row_len(p);
  double* s = (double*)malloc(sizeof(double) * (size_t)(n_rows * (len > 0 ? len : 1)));
  if (!s) return -2;
  orc_score(p, q, K, qI, kI, w, rows, n_rows, s);
  orc_select_f64(s, n_rows, len, len, p->k, idx_out);
  free(s);
  if (p->mode == OMODE_INDEXER) {
    int rc = 0;
    for (int64_t r = 0; r < n_rows; ++r) {
      const int64_t b = rows ? rows[r] : r;
      int64_t* hr = (int64_t*)malloc(sizeof(int64_t) * (size_t)p->Hq);
      for (int64_t h = 0; h < p->Hq; ++h) hr[h] = b * p->Hq + h;
      rc |= orc_attend(p, q, K, V, idx_out + r * p->k, p->k, 0, 3, hr, p->Hq, out + r * p->Hq * p->d);
      free(hr);
    }
    return rc;
  }
  const int64_t unit = (p->mode == OMODE_BLOCK) ? p->block : 0;
  return orc_attend(p, q, K, V, idx_out, p->k, unit, 2, rows, n_rows, out);
}

/*
 * Several query tokens per sequence ("Evolution of Sparse Attention in
 * Long-Context LLMs", section 6: the attention matrix shrinks from "current
 * length x full history" to "current length x K"): M queries per sequence sit
 * at positions L-M .. L-1 of the cache and each attends causally, query t
 * seeing the keys 0 .. L-M+t. Per (b, t, h): exact scores over its L_t =
 * L-M+t+1 visible keys, the top k' = min(k, L_t) in the select order, softmax
 * attention over them. q [B,M,Hq,d]; rows r = (b*M + t)*Hq + h;
 * idx_out [B*M*Hq, k] (ascending, -1 pad), out [B*M*Hq, d].
 */
int orc_decode_mq(const orc_problem* p, int64_t M, const void* q, const void* K, const void* V, double* out,
                  int32_t* idx_out) {
  if (M < 1 || M > p->L || p->k < 1) return -1;
  const int64_t n_rows = (int64_t)p->B * M * p->Hq, G = p->Hq / p->Hkv;
  const double sc = attn_scale(p);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t h = r % p->Hq, bt = r / p->Hq, t = bt % M, b = bt / M, g = h / G;
    const int64_t Lt = p->L - M + t + 1;
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)Lt);
    double* z = (double*)malloc(sizeof(double) * (size_t)Lt);
    for (int64_t i = 0; i < Lt; ++i) {
      double dot = 0;
      for (int64_t c = 0; c < p->d; ++c) dot += ld(q, p->dt, r * p->d + c) * ld(K, p->dt, kv_off(p, b, g, i) + c);
      z[i] = sc * dot;
      tmp[i].v = z[i];
      tmp[i].i = i;
    }
    int32_t* idx = idx_out + r * p->k;
    select_row(tmp, Lt, p->k, idx);
    double M0 = -INFINITY;
    for (int64_t j = 0; j < p->k && idx[j] >= 0; ++j) M0 = z[idx[j]] > M0 ? z[idx[j]] : M0;
    double den = 0;
    for (int64_t c = 0; c < p->d; ++c) out[r * p->d + c] = 0;
    for (int64_t j = 0; j < p->k && idx[j] >= 0; ++j) {
      const double wgt = exp(z[idx[j]] - M0);
      den += wgt;
      for (int64_t c = 0; c < p->d; ++c) out[r * p->d + c] += wgt * ld(V, p->dt, kv_off(p, b, g, idx[j]) + c);
    }
    for (int64_t c = 0; c < p->d; ++c) out[r * p->d + c] /= den;
    free(z);
    free(tmp);
  }
  return 0;
}

/*
 * Two-level (hierarchical) selection, "Sparse Attention Landscape",
 * "Hierarchical Sparse Attention": a coarse score r_j = f_block(q_t, B_j) for
 * every block, the top-K_B blocks kept, token scores s_i = f_token(q_t, k_i)
 * only for the tokens of those blocks, the top-k of them kept, attention over
 * those. Here f_block = <q, mean of the block's keys> (no scale; the mean as
 * in the block variant, the partial last block over its own keys; every one
 * of the m = ceil(L/b) blocks competes) and f_token = scale * <q, k_i>. Both
 * selections use the select order (ties to the lower block / position).
 * All rows: blk_out [B*Hq, KB] (ascending, -1 pad), idx_out [B*Hq, k] token
 * positions (ascending, -1 pad), out [B*Hq, d]; blk_scores [B*Hq, m] or NULL.
 */
int orc_hisa_decode(const orc_problem* p, int64_t KB, const void* q, const void* K, const void* V, double* out,
                    int32_t* idx_out, int32_t* blk_out, double* blk_scores) {
  if (KB < 1 || p->block < 1 || p->k < 1) return -1;
  const int64_t m = n_blocks(p), n_rows = (int64_t)p->B * p->Hq, G = p->Hq / p->Hkv;
  const double sc = attn_scale(p);
  double* means = (double*)malloc(sizeof(double) * (size_t)(p->B * p->Hkv * m * p->d));
  if (!means) return -2;
  orc_block_means(p, K, means);
  int rc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t b = r / p->Hq, h = r % p->Hq, g = h / G;
    double* rj = (double*)malloc(sizeof(double) * (size_t)m);
    for (int64_t j = 0; j < m; ++j) {
      const double* mu = means + ((b * p->Hkv + g) * m + j) * p->d;
      double s = 0;
      for (int64_t c = 0; c < p->d; ++c) s += ld(q, p->dt, (b * p->Hq + h) * p->d + c) * mu[c];
      rj[j] = s;
      if (blk_scores) blk_scores[r * m + j] = s;
    }
    int32_t* blk = blk_out + r * KB;
    orc_select_f64(rj, 1, m, m, KB, blk);
    /* candidate tokens of the kept blocks, ascending (blocks ascend, tokens inside ascend) */
    int64_t nc = 0;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(KB * p->block));
    for (int64_t j = 0; j < KB; ++j) {
      if (blk[j] < 0) continue;
      const int64_t i0 = (int64_t)blk[j] * p->block, i1 = (i0 + p->block < p->L) ? i0 + p->block : p->L;
      for (int64_t i = i0; i < i1; ++i) tok[nc++] = i;
    }
    vi_t* tmp = (vi_t*)malloc(sizeof(vi_t) * (size_t)(nc > 0 ? nc : 1));
    for (int64_t e = 0; e < nc; ++e) {
      tmp[e].v = sc * qk(p, q, K, b, h, tok[e]);
      tmp[e].i = tok[e];  /* ranked by position among equal scores */
    }
    select_row(tmp, nc, p->k, idx_out + r * p->k);
    free(tmp);
    free(tok);
    free(rj);
  }
  free(means);
  if (rc) return rc;
  return orc_attend(p, q, K, V, idx_out, p->k, 0, 0, NULL, n_rows, out);
}

/*
 * Diagnostics of one exact-variant row given its kept set (token positions,
 * -1 ignored). Full softmax P over all L keys, P-hat = P / (1 - tau) on the
 * kept set and 0 elsewhere.
 * res: [0] tau = sum of P off the kept set, [1] TV = 1/2 sum |P - P-hat|,
 *      [2] KL(P-hat || P), [3] entropy of P, [4] boundary gap s_(k') - s_(k'+1)
 *      of the scores in descending order (+inf when k' = L),
 *      [5] cross diameter max ||V_i - V_j|| over i kept, j not kept.
 * o_full [d] = sum P_i V_i, mu_head [d] = sum_kept P-hat_i V_i,
 * mu_tail [d] = sum_not-kept P_i V_i / tau (zeros when tau = 0).
 */
int orc_diag_exact(const orc_problem* p, const void* q, const void* K, const void* V, int64_t row,
                   const int32_t* kept, int64_t n_kept, double* res, double* o_full, double* mu_head,
                   double* mu_tail) {
  const int64_t L = p->L, d = p->d, G = p->Hq / p->Hkv;
  const int64_t b = row / p->Hq, h = row % p->Hq, g = h / G;
  const double sc = attn_scale(p);
  double* s = (double*)malloc(sizeof(double) * (size_t)L);
  double* P = (double*)malloc(sizeof(double) * (size_t)L);
  char* in = (char*)calloc((size_t)L, 1);
  vi_t* srt = (vi_t*)malloc(sizeof(vi_t) * (size_t)L);
  if (!s || !P || !in || !srt) return -2;
  for (int64_t j = 0; j < n_kept; ++j)
    if (kept[j] >= 0 && kept[j] < L) in[kept[j]] = 1;
  double M = -INFINITY;
  for (int64_t i = 0; i < L; ++i) {
    s[i] = sc * qk(p, q, K, b, h, i);
    if (s[i] > M) M = s[i];
    srt[i].v = s[i];
    srt[i].i = i;
  }
  double Z = 0;
  for (int64_t i = 0; i < L; ++i) Z += (P[i] = exp(s[i] - M));
  for (int64_t i = 0; i < L; ++i) P[i] /= Z;
  double tau = 0, keep = 0;
  int64_t nk = 0;
  for (int64_t i = 0; i < L; ++i) {
    if (in[i]) {
      keep += P[i];
      ++nk;
    } else {
      tau += P[i];
    }
  }
  double tv = 0, kl = 0, ent = 0;
  for (int64_t c = 0; c < d; ++c) o_full[c] = mu_head[c] = mu_tail[c] = 0;
  for (int64_t i = 0; i < L; ++i) {
    const double ph = in[i] ? P[i] / keep : 0.0;
    tv += fabs(P[i] - ph);
    if (ph > 0) kl += ph * log(ph / P[i]);
    if (P[i] > 0) ent -= P[i] * log(P[i]);
    const int64_t vo = kv_off(p, b, g, i);
    for (int64_t c = 0; c < d; ++c) {
      const double v = ld(V, p->dt, vo + c);
      o_full[c] += P[i] * v;
      if (in[i]) mu_head[c] += ph * v;
      else mu_tail[c] += P[i] * v;
    }
  }
  for (int64_t c = 0; c < d; ++c) mu_tail[c] = tau > 0 ? mu_tail[c] / tau : 0.0;
  qsort(srt, (size_t)L, sizeof(vi_t), cmp_rank);
  double diam = 0;
  if ((double)nk * (double)(L - nk) <= 2.0e7) {
    /* cross diameter over kept x not-kept pairs (left NaN when too many pairs) */
    for (int64_t i = 0; i < L; ++i) {
      if (!in[i]) continue;
      const int64_t vi = kv_off(p, b, g, i);
      for (int64_t j = 0; j < L; ++j) {
        if (in[j]) continue;
        const int64_t vj = kv_off(p, b, g, j);
        double acc = 0;
        for (int64_t c = 0; c < d; ++c) {
          const double t = ld(V, p->dt, vi + c) - ld(V, p->dt, vj + c);
          acc += t * t;
        }
        if (acc > diam) diam = acc;
      }
    }
  }
  res[0] = tau;
  res[1] = 0.5 * tv;
  res[2] = kl;
  res[3] = ent;
  res[4] = (nk < L && nk > 0) ? srt[nk - 1].v - srt[nk].v : INFINITY;
  res[5] = ((double)nk * (double)(L - nk) <= 2.0e7) ? sqrt(diam) : NAN;
  free(s);
  free(P);
  free(in);
  free(srt);
  return 0;
}

/* threads an OpenMP region of the oracle uses */
int orc_threads(void) { return omp_get_max_threads(); }
