/* Runs every routine of oracle/oracle.c on small seeded inputs (fully random
 * block bytes with finite fp16 fields) so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build reports any out-of-bounds access, overflow
 * or other undefined behaviour; and checks that the factored integer sum
 * agrees with the plain double dequant-and-dot.  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (declared here: the oracle ships no header) */
void orc_quantize_q8_1(const float *x, uint8_t *xq, int64_t rows, int64_t k);
void orc_rms_scale(const float *x, double *r, int64_t rows, int64_t k, double eps);
void orc_qgemv_q8_0(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_q4_k(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_q5_k(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_q6_k(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_q4_0(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_q5_0(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemv_factored(int fmt, const uint8_t *w, const uint8_t *xq, double *y, int64_t n, int64_t k);
void orc_blockdots_q8_0(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t);
void orc_blockdots_q4_k(const uint8_t *, const uint8_t *, int32_t *, int32_t *, int64_t, int64_t);
void orc_blockdots_q5_k(const uint8_t *, const uint8_t *, int32_t *, int32_t *, int64_t, int64_t);
void orc_blockdots_q6_k(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t);
void orc_blockdots_q4_0(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t);
void orc_blockdots_q5_0(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t);
void orc_qgemm_q4_k(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemm_q6_k(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, int64_t, const int64_t *, int64_t);
void orc_qgemm_q8_0(const uint8_t *, const uint8_t *, double *, int64_t, int64_t, int64_t, const int64_t *, int64_t);
void orc_blockdots_q4_k_mmq(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t, int64_t);
void orc_blockdots_q6_k_mmq(const uint8_t *, const uint8_t *, int32_t *, int64_t, int64_t, int64_t);
void orc_router_logits(const float *wr, const float *x, double *logits, int64_t T, int64_t E, int64_t H);
void orc_route_topk(const float *logits, int32_t *ids, double *weights, int64_t T, int64_t E, int64_t K);
void orc_moe_q4_k(const uint8_t *w_gu, const uint8_t *w_down, const uint8_t *xq, const int32_t *ids,
                  const float *weights, int64_t T, int64_t topk, int64_t E, int64_t F, int64_t H, double *gu,
                  uint8_t *hq_out, const uint8_t *hq_in, double *out);

static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
static void fill(uint8_t *p, size_t n) { for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd(); }
/* finite fp16 with exponent in [-14, 2] */
static void put_f16(uint8_t *p) {
  uint16_t h = (uint16_t)(((rnd() & 1) << 15) | ((1 + rnd() % 17) << 10) | (rnd() & 0x3ff));
  memcpy(p, &h, 2);
}
/* random blocks: block bytes, fp16 field offsets */
static uint8_t *blocks(int64_t nblk, int bytes, const int *offs, int noffs) {
  uint8_t *b = malloc((size_t)(nblk * bytes));
  fill(b, (size_t)(nblk * bytes));
  for (int64_t i = 0; i < nblk; ++i)
    for (int j = 0; j < noffs; ++j) put_f16(b + i * bytes + offs[j]);
  return b;
}

static int fails = 0;
static void close_to(const char *what, const double *a, const double *b, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (fabs(a[i] - b[i]) > 1e-9 * (1.0 + fabs(b[i]))) {
      printf("%s: %lld: %.17g vs %.17g\n", what, (long long)i, a[i], b[i]);
      ++fails;
      return;
    }
}

int main(void) {
  const int64_t n = 7, k = 512, nb = k / 32, m = 3;
  float *x = malloc(sizeof(float) * m * k);
  for (int64_t i = 0; i < m * k; ++i) x[i] = (float)((int32_t)rnd() % 20001) / 5000.0f;
  uint8_t *xq = malloc((size_t)(m * nb * 36));
  orc_quantize_q8_1(x, xq, m, k);
  double r[3];
  orc_rms_scale(x, r, m, k, 1e-6);
  const int o0[] = {0}, o01[] = {0, 2}, o6[] = {208};
  struct { int fmt, bytes, per; const int *offs; int no; } F[] = {
      {0, 34, 32, o0, 1}, {1, 144, 256, o01, 2}, {2, 210, 256, o6, 1}, {3, 176, 256, o01, 2},
      {4, 18, 32, o0, 1}, {5, 22, 32, o0, 1}};
  double y[7], yf[7];
  int32_t *D = malloc(sizeof(int32_t) * n * (k / 16)), S[16];
  for (int f = 0; f < 6; ++f) {
    uint8_t *w = blocks(n * (k / F[f].per), F[f].bytes, F[f].offs, F[f].no);
    switch (F[f].fmt) {
      case 0: orc_qgemv_q8_0(w, xq, y, n, k, NULL, 0); orc_blockdots_q8_0(w, xq, D, n, k); break;
      case 1: orc_qgemv_q4_k(w, xq, y, n, k, NULL, 0); orc_blockdots_q4_k(w, xq, D, S, n, k); break;
      case 2: orc_qgemv_q6_k(w, xq, y, n, k, NULL, 0); orc_blockdots_q6_k(w, xq, D, n, k); break;
      case 3: orc_qgemv_q5_k(w, xq, y, n, k, NULL, 0); orc_blockdots_q5_k(w, xq, D, S, n, k); break;
      case 4: orc_qgemv_q4_0(w, xq, y, n, k, NULL, 0); orc_blockdots_q4_0(w, xq, D, n, k); break;
      case 5: orc_qgemv_q5_0(w, xq, y, n, k, NULL, 0); orc_blockdots_q5_0(w, xq, D, n, k); break;
    }
    orc_qgemv_factored(F[f].fmt, w, xq, yf, n, k);
    close_to("factored vs plain", yf, y, n);
    if (F[f].fmt <= 2) {
      double *c = malloc(sizeof(double) * m * n);
      int64_t pairs[4] = {0, 0, m - 1, n - 1};
      if (F[f].fmt == 1) { orc_qgemm_q4_k(w, xq, c, m, n, k, NULL, 0); orc_qgemm_q4_k(w, xq, c, m, n, k, pairs, 2); }
      if (F[f].fmt == 2) { orc_qgemm_q6_k(w, xq, c, m, n, k, NULL, 0); orc_qgemm_q6_k(w, xq, c, m, n, k, pairs, 2); }
      if (F[f].fmt == 0) { orc_qgemm_q8_0(w, xq, c, m, n, k, NULL, 0); orc_qgemm_q8_0(w, xq, c, m, n, k, pairs, 2); }
      int32_t *Dm = malloc(sizeof(int32_t) * m * n * (k / 16));
      if (F[f].fmt == 1) orc_blockdots_q4_k_mmq(w, xq, Dm, m, n, k);
      if (F[f].fmt == 2) orc_blockdots_q6_k_mmq(w, xq, Dm, m, n, k);
      free(Dm);
      free(c);
    }
    free(w);
  }
  /* router and MoE: 3 tokens, 4 experts, F = 256, H = 256, top-2, one id out of range */
  const int64_t T = 3, E = 4, FF = 256, H = 256, K = 2;
  float *wr = malloc(sizeof(float) * E * H), *xt = malloc(sizeof(float) * T * H), lg[12];
  for (int64_t i = 0; i < E * H; ++i) wr[i] = (float)((int32_t)rnd() % 1000) / 1e4f;
  for (int64_t i = 0; i < T * H; ++i) xt[i] = (float)((int32_t)rnd() % 1000) / 100.0f;
  double lgd[12], rw[6];
  orc_router_logits(wr, xt, lgd, T, E, H);
  for (int i = 0; i < 12; ++i) lg[i] = (float)lgd[i];
  int32_t ids[6];
  orc_route_topk(lg, ids, rw, T, E, K);
  ids[3] = (int32_t)E + 1;
  float rwf[6];
  for (int i = 0; i < 6; ++i) rwf[i] = (float)rw[i];
  uint8_t *wgu = blocks(E * 2 * FF * (H / 256), 144, o01, 2), *wdn = blocks(E * H * (FF / 256), 144, o01, 2);
  uint8_t *xtq = malloc((size_t)(T * (H / 32) * 36)), *hq = malloc((size_t)(T * K * (FF / 32) * 36));
  orc_quantize_q8_1(xt, xtq, T, H);
  double *gu = malloc(sizeof(double) * T * K * 2 * FF), *out = malloc(sizeof(double) * T * H);
  orc_moe_q4_k(wgu, wdn, xtq, ids, rwf, T, K, E, FF, H, gu, hq, NULL, out);
  orc_moe_q4_k(wgu, wdn, xtq, ids, rwf, T, K, E, FF, H, NULL, NULL, hq, out);
  free(wr); free(xt); free(wgu); free(wdn); free(xtq); free(hq); free(gu); free(out);
  free(x); free(xq); free(D);
  printf(fails ? "oracle driver: %d failures\n" : "oracle driver: clean%.0d\n", fails);
  return fails != 0;
}
