/*
 * oracle_driver.c -- runs every function of the CPU oracle (oracle/sgqa_oracle.c) on small inputs,
 * edge cases included, so that a build with AddressSanitizer and UndefinedBehaviorSanitizer can
 * flag any out-of-bounds access, use of uninitialised memory or undefined arithmetic in it. Test
 * infrastructure only; compiled together with the oracle source by tests/test_sanitizers.py.
 *
 * Inputs are small integers stored exactly in bf16 (and random FP8 codes), drawn from a fixed
 * linear congruential generator; the driver checks a few exact facts on the way (selection sizes,
 * union counts, coverage range) and exits non-zero on a violation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_f64(uint16_t h);
uint16_t orc_f64_to_bf16(double x);
void orc_compress(int S, int N, int dI, int B, const uint16_t* ki, uint16_t* kbar);
void orc_block_scores(int HI, int dI, const uint16_t* qi_row, const float* w_row, const uint16_t* kbar, int nc,
                      double* s);
void orc_select(int nc, const double* s, int KB, int32_t* out);
void orc_index_topk(int N, int G, int HI, int dI, int B, int KB, const uint16_t* qi, const float* w,
                    const uint16_t* kbar, int nrows, const int32_t* rows, int32_t* topk);
long long orc_scored_pairs(int N, int B);
void orc_union(int N, int G, int B, int KB, int Tq, const int32_t* topk, uint32_t* umask, int32_t* ucount);
void orc_attend(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const uint32_t* umask, int nrows, const int32_t* rows, double* out);
void orc_attend_sel(int N, int Hq, int G, int D, int B, int KB, double scale, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const int32_t* topk, int nrows, const int32_t* rows, double* out);
void orc_attend_bwd(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q, const uint16_t* k,
                    const uint16_t* v, const uint32_t* umask, const uint16_t* dout, double* dq, double* dk,
                    double* dv);
void orc_attend_bwd_part(int N, int Hq, int G, int D, int B, int Tq, double scale, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const uint32_t* umask, const uint16_t* dout, int nr,
                         const int32_t* rows, double* dq_rows, int g0, int key_lo, int key_hi, double* dk_keys,
                         double* dv_keys);
void orc_decode(int S, int L, int Hq, int G, int D, int HI, int dI, int B, int KB, double scale, const uint16_t* q,
                const uint16_t* kc, const uint16_t* vc, const uint16_t* kbar, const uint16_t* qi, const float* w,
                int nseq, const int32_t* seqs, int32_t* topk_out, double* out);
double orc_fp8_e4m3_to_f64(uint8_t b);
void orc_decode_f8(int S, int L, int Hq, int G, int D, int HI, int dI, int B, int KB, double scale,
                   const uint16_t* q, const uint8_t* kc, const uint8_t* vc, const float* kv_scale,
                   const uint16_t* kbar, const uint16_t* qi, const float* w, int nseq, const int32_t* seqs,
                   int32_t* topk_out, double* out);
double orc_coverage(int N, int G, int B, int KB1, int KBB, const int32_t* sel1, const int32_t* selB, int i_min);

static uint64_t lcg_state = 12345;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (uint32_t)(lcg_state >> 33);
}
/* bf16 of a small integer in [-4, 4] (exact). */
static uint16_t small_bf16(void) { return orc_f64_to_bf16((double)((int)(lcg() % 9) - 4)); }
/* bf16 of a value in [-2, 2) with 6 fraction bits (exact). */
static uint16_t frac_bf16(void) { return orc_f64_to_bf16(((int)(lcg() % 256) - 128) / 64.0); }

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}
static uint16_t* fill_small(size_t n) {
  uint16_t* a = (uint16_t*)xmalloc(n * 2);
  for (size_t x = 0; x < n; ++x) a[x] = small_bf16();
  return a;
}
static uint16_t* fill_frac(size_t n) {
  uint16_t* a = (uint16_t*)xmalloc(n * 2);
  for (size_t x = 0; x < n; ++x) a[x] = frac_bf16();
  return a;
}

static int failures = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

/* One prefill chain: compress -> top-k -> union -> attention (+ selection reading, gradient). */
static void prefill_case(int N, int Hq, int G, int B, int KB, int Tq) {
  const int HI = 4, dI = 64, D = 128, NB = N / B, NBc = (N + B - 1) / B;
  const int T = (N + Tq - 1) / Tq, W = (NBc + 31) / 32;
  uint16_t* ki = fill_small((size_t)N * dI);
  uint16_t* qi = fill_small((size_t)N * G * HI * dI);
  float* w = (float*)xmalloc(sizeof(float) * G * HI);
  for (int x = 0; x < G * HI; ++x) w[x] = (float)(1 + lcg() % 2);
  uint16_t* kbar = (uint16_t*)xmalloc((size_t)(NB > 0 ? NB : 1) * dI * 2);
  orc_compress(1, N, dI, B, ki, kbar);
  int32_t* topk = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)G * N * KB);
  orc_index_topk(N, G, HI, dI, B, KB, qi, w, kbar, N, NULL, topk);
  for (int g = 0; g < G; ++g)
    for (int i = 0; i < N; ++i) {
      int n = 0;
      for (int x = 0; x < KB; ++x) n += topk[((size_t)g * N + i) * KB + x] >= 0;
      CHECK(n == (i / B < KB ? i / B : KB));
    }
  /* a row subset, and a score / select pair on the last row */
  int32_t rows[3] = {0, N / 2, N - 1};
  int32_t* sub = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)G * 3 * KB);
  orc_index_topk(N, G, HI, dI, B, KB, qi, w, kbar, 3, rows, sub);
  CHECK(memcmp(sub + 2 * KB, topk + (size_t)(N - 1) * KB, sizeof(int32_t) * KB) == 0);
  const int nc = (N - 1) / B;
  double* s = (double*)xmalloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
  orc_block_scores(HI, dI, qi + (size_t)(N - 1) * G * HI * dI, w, kbar, nc, s);
  int32_t* one = (int32_t*)xmalloc(sizeof(int32_t) * KB);
  orc_select(nc, s, KB, one);
  CHECK(memcmp(one, topk + (size_t)(N - 1) * KB, sizeof(int32_t) * KB) == 0);
  CHECK(orc_scored_pairs(N, B) >= 0);

  uint32_t* umask = (uint32_t*)xmalloc(sizeof(uint32_t) * (size_t)G * T * W);
  int32_t* ucount = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)G * T);
  orc_union(N, G, B, KB, Tq, topk, umask, ucount);
  for (int x = 0; x < G * T; ++x) CHECK(ucount[x] >= 1 && ucount[x] <= NBc);

  uint16_t* q = fill_frac((size_t)N * Hq * D);
  uint16_t* k = fill_frac((size_t)G * N * D);
  uint16_t* v = fill_frac((size_t)G * N * D);
  uint16_t* dout = fill_frac((size_t)N * Hq * D);
  double* out = (double*)xmalloc(sizeof(double) * (size_t)(N > 3 ? N : 3) * Hq * D);  /* N rows or 3 sampled */
  orc_attend(N, Hq, G, D, B, Tq, 0.0, q, k, v, umask, N, NULL, out);
  for (size_t x = 0; x < (size_t)N * Hq * D; ++x) CHECK(isfinite(out[x]));
  orc_attend(N, Hq, G, D, B, Tq, 0.1, q, k, v, umask, 3, rows, out);
  orc_attend_sel(N, Hq, G, D, B, KB, 0.0, q, k, v, topk, N, NULL, out);
  orc_attend_sel(N, Hq, G, D, B, KB, 0.0, q, k, v, topk, 3, rows, out);

  double* dq = (double*)xmalloc(sizeof(double) * (size_t)N * Hq * D);
  double* dk = (double*)xmalloc(sizeof(double) * (size_t)G * N * D);
  double* dv = (double*)xmalloc(sizeof(double) * (size_t)G * N * D);
  orc_attend_bwd(N, Hq, G, D, B, Tq, 0.0, q, k, v, umask, dout, dq, dk, dv);
  double* pq = (double*)xmalloc(sizeof(double) * 3 * Hq * D);
  const int lo = N / 3, hi = N;
  double* pk = (double*)xmalloc(sizeof(double) * (size_t)(hi - lo) * D);
  double* pv = (double*)xmalloc(sizeof(double) * (size_t)(hi - lo) * D);
  orc_attend_bwd_part(N, Hq, G, D, B, Tq, 0.0, q, k, v, umask, dout, 3, rows, pq, G - 1, lo, hi, pk, pv);
  CHECK(memcmp(pq + 2 * Hq * D, dq + (size_t)(N - 1) * Hq * D, sizeof(double) * Hq * D) == 0);
  CHECK(memcmp(pv, dv + ((size_t)(G - 1) * N + lo) * D, sizeof(double) * (size_t)(hi - lo) * D) == 0);
  orc_attend_bwd_part(N, Hq, G, D, B, Tq, 0.0, q, k, v, umask, dout, 0, rows, pq, 0, 0, 0, pk, pv);

  /* coverage of this selection against a token-level one (B = 1) */
  int32_t* sel1 = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)G * N * 2 * KB);
  uint16_t* kbar1 = (uint16_t*)xmalloc((size_t)N * dI * 2);
  orc_compress(1, N, dI, 1, ki, kbar1);
  orc_index_topk(N, G, HI, dI, 1, 2 * KB, qi, w, kbar1, N, NULL, sel1);
  const double cov = orc_coverage(N, G, B, 2 * KB, KB, sel1, topk, 0);
  CHECK(cov >= 0.0 && cov <= 1.0);

  free(ki); free(qi); free(w); free(kbar); free(topk); free(sub); free(s); free(one); free(umask); free(ucount);
  free(q); free(k); free(v); free(dout); free(out); free(dq); free(dk); free(dv); free(pq); free(pk); free(pv);
  free(sel1); free(kbar1);
}

static void decode_case(int S, int L, int Hq, int G, int B, int KB) {
  const int HI = 4, dI = 64, D = 128, NB = L / B;
  uint16_t* q = fill_frac((size_t)S * Hq * D);
  uint16_t* kc = fill_frac((size_t)S * G * L * D);
  uint16_t* vc = fill_frac((size_t)S * G * L * D);
  uint16_t* ki = fill_small((size_t)S * L * dI);
  uint16_t* kbar = (uint16_t*)xmalloc((size_t)S * (NB > 0 ? NB : 1) * dI * 2);
  orc_compress(S, L, dI, B, ki, kbar);
  uint16_t* qi = fill_small((size_t)S * G * HI * dI);
  float* w = (float*)xmalloc(sizeof(float) * G * HI);
  for (int x = 0; x < G * HI; ++x) w[x] = 1.0f;
  int32_t* topk = (int32_t*)xmalloc(sizeof(int32_t) * (size_t)S * G * KB);
  double* out = (double*)xmalloc(sizeof(double) * (size_t)S * Hq * D);
  orc_decode(S, L, Hq, G, D, HI, dI, B, KB, 0.0, q, kc, vc, kbar, qi, w, S, NULL, topk, out);
  int32_t seqs[1] = {S - 1};
  orc_decode(S, L, Hq, G, D, HI, dI, B, KB, 0.0, q, kc, vc, kbar, qi, w, 1, seqs, NULL, out);
  uint8_t* k8 = (uint8_t*)xmalloc((size_t)S * G * L * D);
  uint8_t* v8 = (uint8_t*)xmalloc((size_t)S * G * L * D);
  for (size_t x = 0; x < (size_t)S * G * L * D; ++x) {
    k8[x] = (uint8_t)(lcg() & 0x7Fu) & 0x77u; /* finite codes */
    v8[x] = (uint8_t)(lcg() & 0xFFu) & 0xF7u;
  }
  float* sc = (float*)xmalloc(sizeof(float) * (size_t)S * G * 2);
  for (int x = 0; x < S * G * 2; ++x) sc[x] = 0.5f;
  orc_decode_f8(S, L, Hq, G, D, HI, dI, B, KB, 0.0, q, k8, v8, sc, kbar, qi, w, S, NULL, topk, out);
  for (size_t x = 0; x < (size_t)S * Hq * D; ++x) CHECK(isfinite(out[x]));
  for (int c = 0; c < 256; ++c) (void)orc_fp8_e4m3_to_f64((uint8_t)c);
  free(q); free(kc); free(vc); free(ki); free(kbar); free(qi); free(w); free(topk); free(out); free(k8); free(v8);
  free(sc);
}

int main(void) {
  /* bf16 conversions on special values */
  const double specials[] = {0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 3.4e38, 1e39, -1e39, INFINITY, -INFINITY, NAN};
  for (size_t x = 0; x < sizeof(specials) / sizeof(specials[0]); ++x)
    (void)orc_bf16_to_f64(orc_f64_to_bf16(specials[x]));
  for (uint32_t h = 0; h < 65536; h += 7) (void)orc_f64_to_bf16(orc_bf16_to_f64((uint16_t)h));

  /* prefill: ragged tails, N < B, one tile, block 1 and 64, k covering the context */
  prefill_case(70, 4, 2, 8, 4, 16);
  prefill_case(5, 2, 1, 8, 2, 4);
  prefill_case(1, 2, 1, 1, 1, 1);
  prefill_case(67, 4, 1, 1, 16, 8);
  prefill_case(130, 2, 1, 64, 2, 64);
  prefill_case(48, 4, 2, 4, 32, 48);
  /* decode: L not a multiple of B, L < B, fewer candidates than K_B */
  decode_case(2, 75, 4, 2, 8, 4);
  decode_case(1, 6, 2, 1, 8, 2);
  decode_case(2, 40, 2, 1, 4, 16);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver: all functions ran clean\n");
  return 0;
}
