/*
 * Seeded synthetic inputs for the top-k sparse decode-attention workloads.
 *
 * This module only makes input bytes. It holds none of the method's
 * arithmetic (no scoring, no selection, no softmax): both the CPU oracle and
 * the GPU library receive the bytes it writes.
 *
 * Generator: a counter-based SplitMix64 hash of (seed, tensor id, flat index)
 * gives uniform 53-bit doubles; Box-Muller turns pairs of them into N(0,1).
 * Any element can be regenerated on its own, so rows are filled in parallel.
 * Values are formed in double, rounded once to fp32, then (if asked) to bf16
 * by round-to-nearest-even, or to OCP E4M3FN by round-to-nearest-even with
 * saturation to +-448.
 *
 * Structure planted into the caches (the pages' workloads are long-context
 * decode caches in which a few keys matter much more than the rest):
 *   PLANT_SCALE  - chosen key rows are multiplied by a factor (peaked rows).
 *   PLANT_ALIGN  - chosen key rows are rotated to a fixed cosine with one
 *                  query head of their group, keeping their norm.
 *   PLANT_BLOCK  - every row of chosen blocks is shifted along one query
 *                  head's unit direction.
 * Tensor ids: 0 = q, 1 = K, 2 = V, 3 = planted positions, 4 = indexer query,
 * 5 = indexer keys, 6 = indexer head weights.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FX_F32 0
#define FX_BF16 1
#define FX_E4M3 2

#define PLANT_NONE 0
#define PLANT_SCALE 1
#define PLANT_ALIGN 2
#define PLANT_BLOCK 3

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

static inline uint64_t ctr_hash(uint64_t seed, uint64_t tensor, uint64_t i) {
  return sm64(sm64(sm64(seed) ^ tensor) ^ i);
}

/* uniform in the open interval (0,1) with 53 random bits */
static inline double u53(uint64_t h) { return ((double)(h >> 11) + 0.5) * 0x1.0p-53; }

/* element i of the N(0,1) stream (seed, tensor) */
static inline double normal_at(uint64_t seed, uint64_t tensor, uint64_t i) {
  uint64_t j = i >> 1;
  double u1 = u53(ctr_hash(seed, tensor, 2 * j));
  double u2 = u53(ctr_hash(seed, tensor, 2 * j + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

uint16_t fx_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float fx_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN, max finite 448. */
uint8_t fx_f32_to_e4m3(float f) {
  if (isnan(f)) return 0x7f;
  uint8_t s = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a >= 448.0) return s | 0x7e;
  if (a == 0.0) return s;
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < -6) E = -6;
  double step = ldexp(1.0, E - 3);
  double q = nearbyint(a / step) * step; /* default rounding mode: ties to even */
  if (q == 0.0) return s;
  frexp(q, &e);
  E = e - 1;
  if (E < -6) return s | (uint8_t)(q / ldexp(1.0, -9));
  int mant = (int)(q / ldexp(1.0, E - 3)) - 8;
  return s | (uint8_t)(((E + 7) << 3) | mant);
}

float fx_e4m3_to_f32(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)(s ? -v : v);
}

static void store_val(void* dst, int dtype, int64_t i, double v) {
  float f = (float)v;
  if (dtype == FX_F32) ((float*)dst)[i] = f;
  else if (dtype == FX_BF16) ((uint16_t*)dst)[i] = fx_f32_to_bf16(f);
  else ((uint8_t*)dst)[i] = fx_f32_to_e4m3(f);
}

static double load_val(const void* src, int dtype, int64_t i) {
  if (dtype == FX_F32) return ((const float*)src)[i];
  if (dtype == FX_BF16) return fx_bf16_to_f32(((const uint16_t*)src)[i]);
  return fx_e4m3_to_f32(((const uint8_t*)src)[i]);
}

/* n values of the N(0,1) stream starting at flat index `offset` */
void fx_normal(uint64_t seed, uint64_t tensor, uint64_t offset, int64_t n, int dtype, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) store_val(out, dtype, i, normal_at(seed, tensor, offset + (uint64_t)i));
}

/* n values of U(0,1) with 24 random bits (exact in fp32) */
void fx_uniform_f32(uint64_t seed, uint64_t tensor, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)((double)(ctr_hash(seed, tensor, (uint64_t)i) >> 40) * 0x1.0p-24);
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/* n distinct integers from [0, range), ascending. Stream (seed, 3, stream id). */
int fx_sample_distinct(uint64_t seed, uint64_t stream, int64_t range, int64_t n, int64_t* out) {
  if (n > range || n < 0 || range <= 0) return -1;
  uint8_t* used = (uint8_t*)calloc((size_t)range, 1);
  if (!used) return -2;
  int64_t got = 0;
  uint64_t ctr = 0;
  while (got < n) {
    uint64_t h = ctr_hash(seed, 3, (stream << 32) ^ ctr++);
    int64_t p = (int64_t)(h % (uint64_t)range);
    if (!used[p]) {
      used[p] = 1;
      out[got++] = p;
    }
  }
  free(used);
  qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
  return 0;
}

typedef struct {
  int32_t B, Hq, Hkv, d, L;
  int32_t dtype;       /* FX_F32 or FX_BF16 for q, K and V */
  int32_t plant;       /* PLANT_* */
  int32_t n_plant;     /* per (b, kv head): rows (SCALE, ALIGN) or blocks (BLOCK) */
  int32_t block;       /* block size for PLANT_BLOCK */
  double plant_param;  /* SCALE: factor; ALIGN: cosine; BLOCK: shift length alpha */
  uint64_t seed;
} fx_attn_spec;

/*
 * Fill q [B,Hq,d], K and V [B,Hkv,L,d] (contiguous) per the spec.
 * Planted rows are formed from the unrounded N(0,1) row and the rounded q.
 */
int fx_make_attn(const fx_attn_spec* sp, void* q, void* K, void* V) {
  const int64_t B = sp->B, Hq = sp->Hq, Hkv = sp->Hkv, d = sp->d, L = sp->L;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || L <= 0 || Hq % Hkv) return -1;
  const int64_t G = Hq / Hkv;
  fx_normal(sp->seed, 0, 0, B * Hq * d, sp->dtype, q);
  fx_normal(sp->seed, 1, 0, B * Hkv * L * d, sp->dtype, K);
  fx_normal(sp->seed, 2, 0, B * Hkv * L * d, sp->dtype, V);
  if (sp->plant == PLANT_NONE) return 0;

  const int64_t units = (sp->plant == PLANT_BLOCK) ? (L + sp->block - 1) / sp->block : L;
  if (sp->n_plant > units) return -1;
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(sp->n_plant > 0 ? sp->n_plant : 1));
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* qh = (double*)malloc(sizeof(double) * (size_t)d);
  if (!pos || !row || !qh) return -2;
  int rc = 0;
  for (int64_t b = 0; b < B && rc == 0; ++b) {
    for (int64_t g = 0; g < Hkv && rc == 0; ++g) {
      rc = fx_sample_distinct(sp->seed, (uint64_t)(b * Hkv + g), units, sp->n_plant, pos);
      for (int64_t j = 0; j < sp->n_plant && rc == 0; ++j) {
        const int64_t h = g * G + (j % G);
        double qn = 0;
        for (int64_t c = 0; c < d; ++c) {
          qh[c] = load_val(q, sp->dtype, (b * Hq + h) * d + c);
          qn += qh[c] * qh[c];
        }
        qn = sqrt(qn);
        for (int64_t c = 0; c < d; ++c) qh[c] /= qn;
        if (sp->plant == PLANT_BLOCK) {
          const int64_t i0 = pos[j] * sp->block;
          const int64_t i1 = (i0 + sp->block < L) ? i0 + sp->block : L;
          for (int64_t i = i0; i < i1; ++i) {
            const int64_t base = ((b * Hkv + g) * L + i) * d;
            for (int64_t c = 0; c < d; ++c)
              store_val(K, sp->dtype, base + c,
                        normal_at(sp->seed, 1, (uint64_t)(base + c)) + sp->plant_param * qh[c]);
          }
          continue;
        }
        const int64_t base = ((b * Hkv + g) * L + pos[j]) * d;
        for (int64_t c = 0; c < d; ++c) row[c] = normal_at(sp->seed, 1, (uint64_t)(base + c));
        if (sp->plant == PLANT_SCALE) {
          for (int64_t c = 0; c < d; ++c) store_val(K, sp->dtype, base + c, row[c] * sp->plant_param);
        } else { /* PLANT_ALIGN: same norm, cosine plant_param with q_h */
          double kn = 0, dot = 0;
          for (int64_t c = 0; c < d; ++c) {
            kn += row[c] * row[c];
            dot += row[c] * qh[c];
          }
          kn = sqrt(kn);
          double un = 0;
          for (int64_t c = 0; c < d; ++c) {
            row[c] -= dot * qh[c];
            un += row[c] * row[c];
          }
          un = sqrt(un);
          const double cs = sp->plant_param, sn = sqrt(1.0 - cs * cs);
          for (int64_t c = 0; c < d; ++c)
            store_val(K, sp->dtype, base + c, kn * (cs * qh[c] + sn * row[c] / un));
        }
      }
    }
  }
  free(pos);
  free(row);
  free(qh);
  return rc;
}

/* Indexer inputs: qI [B,HI,dI] and kI [B,L,dI] in E4M3FN, w [B,HI] ~ U(0,1) fp32. */
int fx_make_indexer(uint64_t seed, int32_t B, int32_t HI, int32_t dI, int64_t L, uint8_t* qI, uint8_t* kI,
                    float* w) {
  if (B <= 0 || HI <= 0 || dI <= 0 || L <= 0) return -1;
  fx_normal(seed, 4, 0, (int64_t)B * HI * dI, FX_E4M3, qI);
  fx_normal(seed, 5, 0, (int64_t)B * L * dI, FX_E4M3, kI);
  fx_uniform_f32(seed, 6, (int64_t)B * HI, w);
  return 0;
}

/* bulk converters (used by tests of the encoders) */
void fx_encode(const float* src, int64_t n, int dtype, void* dst) {
  for (int64_t i = 0; i < n; ++i) store_val(dst, dtype, i, src[i]);
}
