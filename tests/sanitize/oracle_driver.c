/* The CPU oracle (oracle/oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every exported function runs on a tiny layer
 * whose buffers are allocated at their exact sizes, with an empty expert,
 * groups not aligned to the 32-blocks, NaN / infinite values for the
 * quantisers and empty calls.  A few invariants are checked on the way
 * (the permutation maps are inverse, combine of the permuted rows with
 * weight 1 is K x).  Exit status 0 and no sanitizer report = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t);
uint16_t oracle_f64_to_bf16(double);
void oracle_bf16_round_array(const double*, uint16_t*, int64_t);
double oracle_e4m3_to_f64(uint8_t);
uint8_t oracle_f64_to_e4m3(double);
double oracle_e8m0_to_f64(uint8_t);
void oracle_route_logits(const uint16_t*, const uint16_t*, const float*, int64_t, int32_t, int32_t, double*);
void oracle_route_topk(const float*, int64_t, int32_t, int32_t, int32_t, int32_t*, float*);
void oracle_permute(const int32_t*, int64_t, int32_t, int32_t, int32_t*, int32_t*, int32_t*, int32_t*);
void oracle_gather_rows(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, uint16_t*);
void oracle_grouped_gemm_rows(const uint16_t*, const uint16_t*, const int32_t*, int32_t, int32_t, int32_t,
                              const int64_t*, int64_t, uint16_t*);
void oracle_gemm_swiglu_rows(const uint16_t*, const uint16_t*, const int32_t*, int32_t, int32_t, int32_t,
                             const int64_t*, int64_t, uint16_t*, uint16_t*);
void oracle_unpermute_combine(const uint16_t*, const float*, const int32_t*, int64_t, int32_t, int32_t, uint16_t*);
void oracle_mxfp8_quantize_rows(const uint16_t*, int64_t, int32_t, uint8_t*, uint8_t*);
void oracle_mxfp8_quantize_cols_grouped(const uint16_t*, int64_t, int32_t, const int32_t*, int32_t, uint8_t*,
                                        uint8_t*);
void oracle_mx_grouped_gemm_rows(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*,
                                 int32_t, int32_t, int32_t, int32_t, const int64_t*, int64_t, uint16_t*);
double oracle_e2m1_to_f64(uint8_t);
uint8_t oracle_f64_to_e2m1(double);
void oracle_mxfp4_quantize_rows(const uint16_t*, int64_t, int32_t, uint8_t*, uint8_t*);
void oracle_mx4_grouped_gemm_rows(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*,
                                  int32_t, int32_t, int32_t, int32_t, const int64_t*, int64_t, uint16_t*);
void oracle_mx_grouped_wgrad(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int32_t*, int32_t,
                             int32_t, int32_t, uint16_t*);
void oracle_combine_backward(const uint16_t*, const uint16_t*, const float*, const int32_t*, int64_t, int32_t,
                             int32_t, uint16_t*, float*);
void oracle_swiglu_backward(const uint16_t*, const uint16_t*, int64_t, int32_t, uint16_t*);
void oracle_grouped_dgrad_rows(const uint16_t*, const uint16_t*, const int32_t*, int32_t, int32_t, int32_t,
                               const int64_t*, int64_t, uint16_t*);
void oracle_grouped_wgrad(const uint16_t*, const uint16_t*, const int32_t*, int32_t, int32_t, int32_t,
                          const int32_t*, int32_t, uint16_t*);

static uint64_t g_state = 12345;
static double draw(void) {   /* uniform in [-2, 2) from a 64-bit LCG */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return ((double)(g_state >> 11) / 9007199254740992.0) * 4.0 - 2.0;
}
static uint16_t* bf16s(size_t n, double scale) {
  uint16_t* p = malloc(n * sizeof *p + 1);
  for (size_t i = 0; i < n; ++i) p[i] = oracle_f64_to_bf16(draw() * scale);
  return p;
}
static void* zalloc(size_t n) { return calloc(n ? n : 1, 1); }
static int g_fail = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); ++g_fail; } } while (0)

int main(void) {
  enum { T = 37, d = 64, E = 5, K = 2, f = 32, M = T * K };
  /* scalar conversions, including the non-finite ones */
  const double specials[] = {0.0, -0.0, 1e-45, -3.5, 448.0, 1e300, INFINITY, -INFINITY, NAN};
  for (size_t i = 0; i < sizeof specials / sizeof *specials; ++i) {
    (void)oracle_f64_to_bf16(specials[i]);
    (void)oracle_f64_to_e4m3(specials[i]);
    (void)oracle_f64_to_e2m1(specials[i]);
  }
  for (int c = 0; c < 256; ++c) { (void)oracle_e4m3_to_f64((uint8_t)c); (void)oracle_e8m0_to_f64((uint8_t)c); }
  for (int c = 0; c < 16; ++c) (void)oracle_e2m1_to_f64((uint8_t)c);
  double dv[3] = {1.0, -2.5, 3e38};
  uint16_t dvb[3];
  oracle_bf16_round_array(dv, dvb, 3);

  /* routing: router scores, then logits with expert E-1 never picked */
  uint16_t* x = bf16s((size_t)T * d, 1.0);
  uint16_t* wr = bf16s((size_t)E * d, 0.125);
  float bias[E] = {0, 0, 0, 0, -1e4f};
  double* sc = malloc(sizeof(double) * T * E);
  oracle_route_logits(x, wr, bias, T, d, E, sc);
  float* lg = malloc(sizeof(float) * T * E);
  for (int i = 0; i < T * E; ++i) lg[i] = (float)sc[i];
  int32_t* ids = malloc(sizeof(int32_t) * M);
  float* w = malloc(sizeof(float) * M);
  oracle_route_topk(lg, T, E, K, 1, ids, w);
  oracle_route_topk(lg, T, E, K, 0, ids, w);
  oracle_route_topk(lg, T, E, K, 1, ids, w);
  oracle_route_topk(lg, 0, E, K, 1, ids, w);   /* no tokens */
  int32_t sizes[E], offs[E + 1];
  int32_t* src = malloc(sizeof(int32_t) * M);
  int32_t* dst = malloc(sizeof(int32_t) * M);
  oracle_permute(ids, T, E, K, sizes, offs, src, dst);
  CHECK(sizes[E - 1] == 0 && offs[E] == M);
  for (int i = 0; i < M; ++i) CHECK(src[dst[i]] == i);
  uint16_t* xp = malloc(sizeof(uint16_t) * M * d);
  oracle_gather_rows(x, src, M, d, K, xp);
  uint16_t* xs = malloc(sizeof(uint16_t) * T * d);
  oracle_unpermute_combine(xp, NULL, dst, T, d, K, xs);
  for (int i = 0; i < T * d; ++i) CHECK(oracle_bf16_to_f64(xs[i]) == K * oracle_bf16_to_f64(x[i]));

  /* forward GEMMs over every row, and over a row list */
  int64_t* rows = malloc(sizeof(int64_t) * M);
  for (int i = 0; i < M; ++i) rows[i] = i;
  uint16_t* w1 = bf16s((size_t)E * 2 * f * d, 0.125);
  uint16_t* w2 = bf16s((size_t)E * d * f, 0.18);
  uint16_t* h = malloc(sizeof(uint16_t) * M * f);
  uint16_t* gu = malloc(sizeof(uint16_t) * M * 2 * f);
  oracle_gemm_swiglu_rows(xp, w1, sizes, E, f, d, rows, M, h, gu);
  oracle_gemm_swiglu_rows(xp, w1, sizes, E, f, d, rows + 3, 5, h, NULL);
  uint16_t* yp = malloc(sizeof(uint16_t) * M * d);
  oracle_grouped_gemm_rows(h, w2, sizes, E, d, f, rows, M, yp);
  uint16_t* y = malloc(sizeof(uint16_t) * T * d);
  oracle_unpermute_combine(yp, w, dst, T, d, K, y);

  /* backward */
  uint16_t* dy = bf16s((size_t)T * d, 1.0);
  uint16_t* dyp = malloc(sizeof(uint16_t) * M * d);
  float* dw = malloc(sizeof(float) * M);
  oracle_combine_backward(dy, yp, w, dst, T, d, K, dyp, dw);
  uint16_t* dh = malloc(sizeof(uint16_t) * M * f);
  oracle_grouped_dgrad_rows(dyp, w2, sizes, E, d, f, rows, M, dh);
  uint16_t* dgu = malloc(sizeof(uint16_t) * M * 2 * f);
  oracle_swiglu_backward(gu, dh, M, f, dgu);
  uint16_t* dxp = malloc(sizeof(uint16_t) * M * d);
  oracle_grouped_dgrad_rows(dgu, w1, sizes, E, 2 * f, d, rows, M, dxp);
  uint16_t* dw2 = malloc(sizeof(uint16_t) * E * d * f);
  oracle_grouped_wgrad(dyp, h, sizes, E, d, f, NULL, E, dw2);
  for (int i = 0; i < d * f; ++i) CHECK(dw2[(size_t)(E - 1) * d * f + i] == 0);
  int32_t pick[2] = {E - 1, 0};
  uint16_t* dw1 = malloc(sizeof(uint16_t) * 2 * 2 * f * d);
  oracle_grouped_wgrad(dgu, xp, sizes, E, 2 * f, d, pick, 2, dw1);

  /* MXFP8: rows, grouped columns (groups of 37 and 0 and 37 rows), GEMMs, wgrad */
  uint16_t* xn = bf16s((size_t)M * d, 1.0);
  xn[5] = 0x7FC0; xn[d + 7] = 0xFF80; xn[2 * d + 40] = 0x7F80;   /* NaN, -inf, +inf */
  uint8_t* q0 = malloc((size_t)M * d);
  uint8_t* s0 = malloc((size_t)M * d / 32);
  oracle_mxfp8_quantize_rows(xn, M, d, q0, s0);
  CHECK(s0[0] == 0xFF && s0[d / 32] == 0xFF);
  int32_t gs[3] = {37, 0, 37};
  const int nb = (37 + 31) / 32 * 2;
  uint8_t* q1 = zalloc((size_t)M * d);
  uint8_t* s1 = zalloc((size_t)nb * d);
  oracle_mxfp8_quantize_cols_grouped(xn, M, d, gs, 3, q1, s1);
  uint8_t* wq = malloc((size_t)E * 2 * f * d);
  uint8_t* ws = malloc((size_t)E * 2 * f * d / 32);
  oracle_mxfp8_quantize_rows(w1, (int64_t)E * 2 * f, d, wq, ws);
  oracle_mxfp8_quantize_rows(xp, M, d, q0, s0);
  oracle_mx_grouped_gemm_rows(q0, s0, wq, ws, sizes, E, 2 * f, d, 1, rows, M, h);
  oracle_mx_grouped_gemm_rows(q0, s0, wq, ws, sizes, E, 2 * f, d, 0, rows, M, gu);
  uint8_t* aq = zalloc((size_t)M * d);
  uint8_t* as = zalloc((size_t)M * d);
  uint8_t* bq = zalloc((size_t)M * f);
  uint8_t* bs = zalloc((size_t)M * f);
  oracle_mxfp8_quantize_cols_grouped(dyp, M, d, sizes, E, aq, as);
  oracle_mxfp8_quantize_cols_grouped(h, M, f, sizes, E, bq, bs);
  oracle_mx_grouped_wgrad(aq, as, bq, bs, sizes, E, d, f, dw2);

  /* MXFP4 */
  uint8_t* c4 = malloc((size_t)M * d);
  uint8_t* s4 = malloc((size_t)M * d / 32);
  oracle_mxfp4_quantize_rows(xn, M, d, c4, s4);
  oracle_mxfp4_quantize_rows(xp, M, d, c4, s4);
  uint8_t* w4 = malloc((size_t)E * 2 * f * d);
  uint8_t* w4s = malloc((size_t)E * 2 * f * d / 32);
  oracle_mxfp4_quantize_rows(w1, (int64_t)E * 2 * f, d, w4, w4s);
  oracle_mx4_grouped_gemm_rows(c4, s4, w4, w4s, sizes, E, 2 * f, d, 1, rows, M, h);

  free(x); free(wr); free(sc); free(lg); free(ids); free(w); free(src); free(dst); free(xp); free(xs);
  free(rows); free(w1); free(w2); free(h); free(gu); free(yp); free(y); free(dy); free(dyp); free(dw);
  free(dh); free(dgu); free(dxp); free(dw2); free(dw1); free(xn); free(q0); free(s0); free(q1); free(s1);
  free(wq); free(ws); free(aq); free(as); free(bq); free(bs); free(c4); free(s4); free(w4); free(w4s);
  printf("%s: %d checks failed\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
