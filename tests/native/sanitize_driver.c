/*
 * Sanitizer driver for the CPU oracle (oracle/oracle.c) and the seeded input
 * generator (fixtures/gen.c): test infrastructure only.
 *
 * Built by tests/test_sanitizers.py with gcc, AddressSanitizer and
 * UndefinedBehaviorSanitizer (runtimes linked statically, every report
 * fatal), together with both sources. It calls every exported function of
 * both on small inputs that reach their edge cases: ragged and partial
 * blocks, k above the row length, empty rows, NaN / +-0 / +-inf scores,
 * every kept-list mode, strided caches. A sanitizer report aborts the
 * process; otherwise a few invariants are checked and it prints "ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* declarations of the two libraries (the same layouts as their sources) */
typedef struct {
  int32_t B, Hq, Hkv, d, L, k;
  int64_t sb, sh, sl;
  int32_t dt;
  double scale;
  int32_t mode;
  int32_t block;
  int32_t HI, dI;
} orc_problem;

typedef struct {
  int32_t B, Hq, Hkv, d, L;
  int32_t dtype, plant, n_plant, block;
  double plant_param;
  uint64_t seed;
} fx_attn_spec;

int orc_score(const orc_problem*, const void*, const void*, const void*, const void*, const float*, const int64_t*,
              int64_t, double*);
int orc_block_means(const orc_problem*, const void*, double*);
int orc_select_f64(const double*, int64_t, int64_t, int64_t, int64_t, int32_t*);
int orc_select_f32(const float*, int64_t, int64_t, int64_t, int64_t, int32_t*);
int orc_select_adaptive_f32(const float*, int64_t, int64_t, int64_t, double, int64_t, int64_t, int32_t*, int32_t*,
                            double*);
int orc_select_adaptive_f64(const double*, int64_t, int64_t, int64_t, double, int64_t, int64_t, int32_t*, int32_t*,
                            double*);
int orc_attend(const orc_problem*, const void*, const void*, const void*, const int32_t*, int64_t, int64_t, int32_t,
               const int64_t*, int64_t, double*);
int orc_decode(const orc_problem*, const void*, const void*, const void*, const void*, const void*, const float*,
               const int64_t*, int64_t, double*, int32_t*);
int orc_decode_mq(const orc_problem*, int64_t, const void*, const void*, const void*, double*, int32_t*);
int orc_hisa_decode(const orc_problem*, int64_t, const void*, const void*, const void*, double*, int32_t*, int32_t*,
                    double*);
int orc_diag_exact(const orc_problem*, const void*, const void*, const void*, int64_t, const int32_t*, int64_t,
                   double*, double*, double*, double*);
void orc_encode_e4m3(const float*, int64_t, uint8_t*);
void orc_decode_buf(int, const void*, int64_t, double*);
double orc_dec_bf16(uint16_t);
double orc_dec_e4m3(uint8_t);
int orc_threads(void);

void fx_normal(uint64_t, uint64_t, uint64_t, int64_t, int, void*);
void fx_uniform_f32(uint64_t, uint64_t, int64_t, float*);
int fx_sample_distinct(uint64_t, uint64_t, int64_t, int64_t, int64_t*);
int fx_make_attn(const fx_attn_spec*, void*, void*, void*);
int fx_make_indexer(uint64_t, int32_t, int32_t, int32_t, int64_t, uint8_t*, uint8_t*, float*);
void fx_encode(const float*, int64_t, int, void*);
uint16_t fx_f32_to_bf16(float);
float fx_bf16_to_f32(uint16_t);
uint8_t fx_f32_to_e4m3(float);
float fx_e4m3_to_f32(uint8_t);

static int failures = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

/* exact sizes, so an off-by-one read or write lands in a redzone */
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

static void check_ascending(const int32_t* idx, int64_t k, int64_t kk, int64_t n) {
  for (int64_t j = 0; j < k; ++j) {
    if (j < kk) CHECK(idx[j] >= 0 && idx[j] < n && (j == 0 || idx[j] > idx[j - 1]));
    else CHECK(idx[j] == -1);
  }
}

/* exact variant, dtype dt, with cache strides (capacity Lcap, row pad) */
static void exact_case(int dt, int B, int Hq, int Hkv, int d, int L, int k, int Lcap, int pad, int plant) {
  const size_t es = dt == 0 ? 4 : 2;
  const int row = d + pad;
  fx_attn_spec sp = {B, Hq, Hkv, d, L, dt, plant, plant == 0 ? 0 : 3, 0, plant == 1 ? 3.0 : 0.5, 7};
  void* q = xmalloc(es * (size_t)B * Hq * d);
  void* K = xmalloc(es * (size_t)B * Hkv * L * d);
  void* V = xmalloc(es * (size_t)B * Hkv * L * d);
  CHECK(fx_make_attn(&sp, q, K, V) == 0);
  /* strided copies: rows of `row` elements, Lcap positions per head; only [:L, :d] written */
  const size_t nbig = (size_t)B * Hkv * Lcap * row;
  char* Ks = (char*)xmalloc(es * nbig);
  char* Vs = (char*)xmalloc(es * nbig);
  memset(Ks, 0, es * nbig);
  memset(Vs, 0, es * nbig);
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int i = 0; i < L; ++i) {
        const size_t src = (((size_t)b * Hkv + g) * L + i) * d, dst = (((size_t)b * Hkv + g) * Lcap + i) * row;
        memcpy(Ks + es * dst, (char*)K + es * src, es * d);
        memcpy(Vs + es * dst, (char*)V + es * src, es * d);
      }
  orc_problem p = {B, Hq, Hkv, d, L, k, (int64_t)Hkv * Lcap * row, (int64_t)Lcap * row, row, dt, 0.0, 0, 0, 0, 0};
  const int64_t rows = (int64_t)B * Hq;
  double* s = (double*)xmalloc(sizeof(double) * rows * L);
  CHECK(orc_score(&p, q, Ks, NULL, NULL, NULL, NULL, rows, s) == 0);
  int32_t* idx = (int32_t*)xmalloc(sizeof(int32_t) * rows * k);
  double* out = (double*)xmalloc(sizeof(double) * rows * d);
  CHECK(orc_decode(&p, q, Ks, Vs, NULL, NULL, NULL, NULL, rows, out, idx) == 0);
  const int64_t kk = k < L ? k : L;
  for (int64_t r = 0; r < rows; ++r) check_ascending(idx + r * k, k, kk, L);
  /* a subset of rows through `rows`, and list modes 0..3 */
  int64_t sub[2] = {rows - 1, 0};
  double* o2 = (double*)xmalloc(sizeof(double) * 2 * d);
  CHECK(orc_attend(&p, q, Ks, Vs, idx, k, 0, 0, sub, 2, o2) == 0);
  /* list mode 2: one list per entry of `rows` */
  int32_t* two = (int32_t*)xmalloc(sizeof(int32_t) * 2 * k);
  memcpy(two, idx + (rows - 1) * k, sizeof(int32_t) * k);
  memcpy(two + k, idx, sizeof(int32_t) * k);
  CHECK(orc_attend(&p, q, Ks, Vs, two, k, 0, 2, sub, 2, o2) == 0);
  free(two);
  CHECK(orc_attend(&p, q, Ks, Vs, idx, k, 0, 3, NULL, rows, out) == 0);
  CHECK(orc_attend(&p, q, Ks, Vs, idx, k, 0, 1, NULL, rows, out) == 0);
  /* diagnostics of every row (keeps the cross diameter where pairs are few) */
  double res[6];
  double* of = (double*)xmalloc(sizeof(double) * d * 3);
  for (int64_t r = 0; r < rows; ++r) {
    CHECK(orc_diag_exact(&p, q, Ks, Vs, r, idx + r * k, k, res, of, of + d, of + 2 * d) == 0);
    CHECK(fabs(res[0] - res[1]) < 1e-9);
  }
  /* several queries: the last M positions, causal */
  const int M = L >= 3 ? 3 : 1;
  void* qm = xmalloc(es * (size_t)B * M * Hq * d);
  fx_normal(9, 0, 0, (int64_t)B * M * Hq * d, dt, qm);
  int32_t* idxm = (int32_t*)xmalloc(sizeof(int32_t) * rows * M * k);
  double* outm = (double*)xmalloc(sizeof(double) * rows * M * d);
  CHECK(orc_decode_mq(&p, M, qm, Ks, Vs, outm, idxm) == 0);
  /* two levels, blocks of 16 with a partial last block */
  p.block = 16;
  const int64_t m = (L + 15) / 16, KB = m > 3 ? 3 : m;
  double* bsc = (double*)xmalloc(sizeof(double) * rows * m);
  int32_t* blk = (int32_t*)xmalloc(sizeof(int32_t) * rows * KB);
  CHECK(orc_hisa_decode(&p, KB, q, Ks, Vs, out, idx, blk, bsc) == 0);
  double* means = (double*)xmalloc(sizeof(double) * B * Hkv * m * d);
  CHECK(orc_block_means(&p, Ks, means) == 0);
  free(means);
  free(bsc);
  free(blk);
  free(qm);
  free(idxm);
  free(outm);
  free(of);
  free(o2);
  free(out);
  free(idx);
  free(s);
  free(Ks);
  free(Vs);
  free(q);
  free(K);
  free(V);
}

static void block_case(int B, int Hq, int Hkv, int d, int L, int bsz, int k) {
  const int nb = (L + bsz - 1) / bsz;
  fx_attn_spec sp = {B, Hq, Hkv, d, L, 1, 3, nb < 2 ? nb : 2, bsz, 0.8, 4};
  uint16_t* q = (uint16_t*)xmalloc(2 * (size_t)B * Hq * d);
  uint16_t* K = (uint16_t*)xmalloc(2 * (size_t)B * Hkv * L * d);
  uint16_t* V = (uint16_t*)xmalloc(2 * (size_t)B * Hkv * L * d);
  CHECK(fx_make_attn(&sp, q, K, V) == 0);
  orc_problem p = {B, Hq, Hkv, d, L, k, (int64_t)Hkv * L * d, (int64_t)L * d, d, 1, 0.0, 1, bsz, 0, 0};
  const int64_t rows = (int64_t)B * Hq, m = (L + bsz - 1) / bsz;
  double* s = (double*)xmalloc(sizeof(double) * rows * (m > 1 ? m - 1 : 1));
  CHECK(orc_score(&p, q, K, NULL, NULL, NULL, NULL, rows, s) == 0);
  int32_t* idx = (int32_t*)xmalloc(sizeof(int32_t) * rows * k);
  double* out = (double*)xmalloc(sizeof(double) * rows * d);
  CHECK(orc_decode(&p, q, K, V, NULL, NULL, NULL, NULL, rows, out, idx) == 0);
  CHECK(orc_attend(&p, q, K, V, idx, k, bsz, 0, NULL, rows, out) == 0);
  free(s);
  free(idx);
  free(out);
  free(q);
  free(K);
  free(V);
}

static void indexer_case(int L, int HI, int dI, int k) {
  const int B = 1, Hq = 4, Hkv = 2, d = 64;
  fx_attn_spec sp = {B, Hq, Hkv, d, L, 1, 0, 0, 0, 0.0, 5};
  uint16_t* q = (uint16_t*)xmalloc(2 * (size_t)B * Hq * d);
  uint16_t* K = (uint16_t*)xmalloc(2 * (size_t)B * Hkv * L * d);
  uint16_t* V = (uint16_t*)xmalloc(2 * (size_t)B * Hkv * L * d);
  CHECK(fx_make_attn(&sp, q, K, V) == 0);
  uint8_t* qI = (uint8_t*)xmalloc((size_t)B * HI * dI);
  uint8_t* kI = (uint8_t*)xmalloc((size_t)B * L * dI);
  float* w = (float*)xmalloc(sizeof(float) * B * HI);
  CHECK(fx_make_indexer(5, B, HI, dI, L, qI, kI, w) == 0);
  orc_problem p = {B, Hq, Hkv, d, L, k, (int64_t)Hkv * L * d, (int64_t)L * d, d, 1, 0.0, 2, 0, HI, dI};
  double* s = (double*)xmalloc(sizeof(double) * B * L);
  CHECK(orc_score(&p, NULL, NULL, qI, kI, w, NULL, B, s) == 0);
  int32_t* idx = (int32_t*)xmalloc(sizeof(int32_t) * B * k);
  double* out = (double*)xmalloc(sizeof(double) * B * Hq * d);
  CHECK(orc_decode(&p, q, K, V, qI, kI, w, NULL, B, out, idx) == 0);
  check_ascending(idx, k, k < L ? k : L, L);
  free(s);
  free(idx);
  free(out);
  free(qI);
  free(kI);
  free(w);
  free(q);
  free(K);
  free(V);
}

static void select_edges(void) {
  /* NaN, +-0, +-inf, ties; every k from 1 to len + 2; an empty row */
  const int n = 11;
  float v[11] = {1.f, NAN, -0.f, 0.f, INFINITY, -INFINITY, 1.f, NAN, 2.f, -1.f, 2.f};
  double vd[11];
  for (int i = 0; i < n; ++i) vd[i] = v[i];
  for (int k = 1; k <= n + 2; ++k) {
    int32_t* idx = (int32_t*)xmalloc(sizeof(int32_t) * k);
    int32_t* idx2 = (int32_t*)xmalloc(sizeof(int32_t) * k);
    CHECK(orc_select_f32(v, 1, n, n, k, idx) == 0);
    CHECK(orc_select_f64(vd, 1, n, n, k, idx2) == 0);
    CHECK(memcmp(idx, idx2, sizeof(int32_t) * k) == 0);
    check_ascending(idx, k, k < n ? k : n, n);
    int32_t kk = 0;
    double tau = 0;
    CHECK(orc_select_adaptive_f32(v, 1, n, n, 0.1, 1, k, idx, &kk, &tau) == 0);
    CHECK(orc_select_adaptive_f64(vd, 1, n, n, 0.5, 0, k, idx2, &kk, &tau) == 0);
    free(idx);
    free(idx2);
  }
  int32_t e[3];
  CHECK(orc_select_f32(v, 1, 0, 0, 3, e) == 0);
  CHECK(e[0] == -1 && e[2] == -1);
  int32_t kk = 0;
  double tau = 0;
  float nanrow[4] = {NAN, NAN, NAN, NAN};
  CHECK(orc_select_adaptive_f32(nanrow, 1, 4, 4, 0.1, 0, 3, e, &kk, &tau) == 0);
  CHECK(kk == 1 && isnan(tau));
  CHECK(orc_select_f32(v, 1, n, n, 0, e) != 0); /* bad k is refused */
}

static void codes(void) {
  float x[260];
  for (int i = 0; i < 256; ++i) x[i] = (float)orc_dec_e4m3((uint8_t)i);
  x[256] = 1e30f;
  x[257] = -INFINITY;
  x[258] = NAN;
  x[259] = -0.f;
  uint8_t c[260], c2[260];
  orc_encode_e4m3(x, 260, c);
  fx_encode(x, 260, 2, c2);
  for (int i = 0; i < 260; ++i)
    if (!isnan(x[i])) CHECK(c[i] == c2[i]);
  double dd[260];
  orc_decode_buf(2, c, 260, dd);
  uint16_t h[260];
  fx_encode(x, 260, 1, h);
  orc_decode_buf(1, h, 260, dd);
  for (int i = 0; i < 256; ++i)
    if (!isnan(x[i])) CHECK((double)fx_bf16_to_f32(fx_f32_to_bf16(x[i])) == orc_dec_bf16(fx_f32_to_bf16(x[i])));
  for (int i = 0; i < 256; ++i) CHECK(isnan(fx_e4m3_to_f32((uint8_t)i)) || fx_f32_to_e4m3(fx_e4m3_to_f32((uint8_t)i)) == (uint8_t)i || (i & 0x7f) == 0);
  float u[37];
  fx_uniform_f32(3, 6, 37, u);
  for (int i = 0; i < 37; ++i) CHECK(u[i] > 0.f && u[i] < 1.f);
  int64_t pos[50];
  CHECK(fx_sample_distinct(3, 3, 50, 50, pos) == 0);
  for (int i = 0; i < 50; ++i) CHECK(pos[i] == i);
  CHECK(fx_sample_distinct(3, 3, 10, 11, pos) != 0);
}

int main(void) {
  CHECK(orc_threads() >= 1);
  select_edges();
  codes();
  exact_case(0, 1, 1, 1, 64, 1001, 64, 1100, 4, 1);   /* fp32, padded rows, k < L */
  exact_case(1, 2, 4, 2, 32, 37, 50, 40, 8, 2);       /* bf16, k > L, partial block */
  exact_case(1, 1, 8, 2, 128, 300, 17, 300, 0, 2);    /* bf16, G = 4 */
  exact_case(0, 1, 2, 1, 16, 3, 1, 3, 0, 0);          /* tiny: L = 3, k = 1 */
  block_case(2, 4, 2, 32, 64 * 9 + 5, 64, 3);         /* partial last block */
  block_case(1, 2, 1, 32, 64, 64, 2);                 /* one block: nothing competes */
  indexer_case(777, 4, 64, 50);
  indexer_case(40, 3, 128, 64);                       /* k > L */
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
