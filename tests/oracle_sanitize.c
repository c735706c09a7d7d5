/*
 * Drives every exported function of the CPU oracle (oracle/elmo_oracle.c) on small inputs, edge
 * cases included, so that a build with -fsanitize=address,undefined checks its memory accesses and
 * arithmetic for undefined behaviour. It also checks a few properties that hold for any input
 * (codec round trips, stochastic rounding brackets, the step's weight half, top-k order), and exits
 * non-zero on the first failure. Test infrastructure only.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/elmo_oracle.h"

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      exit(1);                                                       \
    }                                                                \
  } while (0)

static uint64_t lcg_state = 88172645463325252ull;
static uint32_t rnd32(void) {
  lcg_state ^= lcg_state << 13; lcg_state ^= lcg_state >> 7; lcg_state ^= lcg_state << 17;
  return (uint32_t)(lcg_state >> 16);
}
static double rnd_unit(void) { return (rnd32() + 0.5) / 4294967296.0; }
static double rnd_gauss(void) { return sqrt(-2.0 * log(rnd_unit())) * cos(6.283185307179586 * rnd_unit()); }

static void codecs(void) {
  for (uint32_t c = 0; c < 65536; ++c) {
    double v = orc_bf16_value((uint16_t)c);
    if (!isnan(v)) CHECK(orc_bf16_rne((float)v) == (uint16_t)c || (v == 0.0));
  }
  for (uint32_t c = 0; c < 256; ++c) {
    double v = orc_e4m3_value((uint8_t)c);
    if (!isnan(v)) CHECK(orc_e4m3_rne_sat(v) == (uint8_t)c || v == 0.0);
  }
  CHECK(orc_e4m3_rne_sat(1e9) == 0x7E && orc_e4m3_rne_sat(-INFINITY) == 0xFE);
  CHECK((orc_e4m3_rne_sat(NAN) & 0x7F) == 0x7F);
  float xs[5] = {1.0f, -3.1f, 1e-30f, 448.5f, NAN};
  uint16_t b[5]; double xd[5]; uint8_t e[5];
  orc_bf16_rne_array(xs, b, 5);
  for (int i = 0; i < 5; ++i) xd[i] = xs[i];
  orc_e4m3_rne_sat_array(xd, e, 5);
  CHECK(b[0] == 0x3F80 && e[0] == 0x38);
}

static void rounding(void) {
  float ts[6] = {0.0213f, -0.0213f, 1e-3f, 447.9f, 3.0e-3f, -1e-40f};
  for (int i = 0; i < 6; ++i) {
    uint32_t up_b = 0, up_e = 0;
    uint16_t lo_b = orc_sr_bf16(ts[i], 0);
    uint8_t lo_e = orc_sr_e4m3(ts[i], 0);
    for (uint32_t r = 0; r < 65536; ++r) {
      up_b += orc_sr_bf16(ts[i], r) != lo_b;
      up_e += orc_sr_e4m3(ts[i], r) != lo_e;
    }
    CHECK(up_b < 65536 && up_e < 65536);
  }
  CHECK((orc_sr_bf16(NAN, 5) & 0x7FFF) > 0x7F80 && (orc_sr_e4m3(NAN, 5) & 0x7F) == 0x7F);
  CHECK(orc_sr_e4m3(1e6f, 0) == 0x7E && orc_sr_bf16(INFINITY, 77) == 0x7F80);
  float t[4] = {0.5f, 0.75f, -2.5f, 1e-8f};
  uint32_t r[4] = {0, 1, 65535, 32768};
  uint16_t ob[4]; uint8_t oe[4];
  orc_sr_bf16_array(t, r, ob, 4);
  orc_sr_e4m3_array(t, r, oe, 4);
  CHECK(ob[0] == 0x3F00 && oe[0] == 0x30);
  uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4];
  orc_philox4x32(ctr, key, 10, out);
  CHECK(out[0] == 0x6627E8D5u);
  uint32_t draws[20];
  orc_r16_array(7, 3, (1ull << 33) - 4, draws, 20);
  for (int i = 0; i < 20; ++i) CHECK(draws[i] == orc_r16(7, 3, (1ull << 33) - 4 + (uint64_t)i) && draws[i] < 65536);
}

/* a tiny step in both formats, with empty, duplicated and unsorted label rows */
static void step(int wfmt) {
  enum { B = 5, D = 16, L = 37 };
  size_t esz = wfmt == ORC_W_BF16 ? 2 : 1;
  uint8_t* W = malloc(esz * L * D);
  uint8_t* W2 = malloc(esz * L * D);
  uint8_t* Wu = malloc(esz * L * D);
  uint16_t X[B * D];
  for (int i = 0; i < L * D; ++i) {
    double v = 0.2 * rnd_gauss();
    if (wfmt == ORC_W_BF16) ((uint16_t*)W)[i] = orc_bf16_rne((float)v);
    else W[i] = orc_e4m3_rne_sat(v);
  }
  for (int i = 0; i < B * D; ++i) X[i] = orc_bf16_rne((float)(0.5 * rnd_gauss()));
  int32_t row_ptr[B + 1] = {0, 3, 3, 6, 7, 9};
  int32_t ids[9] = {36, 0, 5, 5, 12, 5, 0, 36, 2};
  float dX[B * D], Z[B * L], T[L * D], dXr[2 * D], Zs[B * 3], Tr[3 * D];
  uint16_t G[B * L], Gr[B * 3];
  double loss = 0.0;
  memcpy(W2, W, esz * L * D);
  CHECK(orc_step(wfmt, W2, L, D, X, B, row_ptr, ids, 0.05f, 9, 2, dX, &loss, Z, G, 2) == ORC_OK);
  CHECK(isfinite(loss) && loss > 0.0);
  CHECK(orc_update_from_g(wfmt, W, L, D, X, B, G, 0.05f, 9, 2, Wu, T, 1) == ORC_OK);
  CHECK(memcmp(Wu, W2, esz * L * D) == 0);
  int64_t js[3] = {0, 17, 36};
  uint8_t* Wr = malloc(esz * 3 * D);
  CHECK(orc_update_rows(wfmt, W, L, D, X, B, row_ptr, ids, 0.05f, 9, 2, js, 3, Wr, Gr, Tr, 1) == ORC_OK);
  for (int i = 0; i < 3; ++i) {
    CHECK(memcmp(Wr + esz * i * D, W2 + esz * js[i] * D, esz * D) == 0);
    CHECK(memcmp(Tr + i * D, T + js[i] * D, sizeof(float) * D) == 0);
    for (int b = 0; b < B; ++b) CHECK(Gr[b * 3 + i] == G[b * L + js[i]]);
  }
  CHECK(orc_update_rows_from_g(wfmt, W, L, D, X, B, Gr, 0.05f, 9, 2, js, 3, Wr, 1) == ORC_OK);
  CHECK(memcmp(Wr + esz * D, W2 + esz * 17 * D, esz * D) == 0);
  CHECK(orc_logits(wfmt, W, L, D, X, B, js, 3, Zs, 1) == ORC_OK);
  for (int b = 0; b < B; ++b) CHECK(Zs[b * 3 + 1] == Z[b * L + 17]);
  int32_t bs[2] = {0, B - 1};
  CHECK(orc_dx_rows(wfmt, W, L, D, X, B, row_ptr, ids, bs, 2, dXr, 3) == ORC_OK);
  for (int k = 0; k < D; ++k) CHECK(fabsf(dXr[D + k] - dX[(B - 1) * D + k]) <= 1e-6f * (1.0f + fabsf(dX[(B - 1) * D + k])));
  /* top-k with k = L: a full ranking */
  int32_t idx[2 * L];
  float sc[2 * L];
  CHECK(orc_topk(wfmt, W, L, D, X, 2, L, idx, sc, 2) == ORC_OK);
  for (int i = 0; i + 1 < L; ++i) CHECK(sc[i] > sc[i + 1] || (sc[i] == sc[i + 1] && idx[i] < idx[i + 1]));
  /* errors: a label outside [0, L), a null pointer, a bad format */
  int32_t bad[9];
  memcpy(bad, ids, sizeof bad);
  bad[4] = L;
  memcpy(W2, W, esz * L * D);
  CHECK(orc_step(wfmt, W2, L, D, X, B, row_ptr, bad, 0.05f, 9, 2, dX, NULL, NULL, NULL, 1) == ORC_EINVAL);
  CHECK(orc_step(wfmt, W2, L, D, X, B, row_ptr, ids, 0.05f, 9, 2, NULL, NULL, NULL, NULL, 1) == ORC_EINVAL);
  CHECK(orc_step(7, W2, L, D, X, B, row_ptr, ids, 0.05f, 9, 2, dX, NULL, NULL, NULL, 1) == ORC_EINVAL);
  CHECK(orc_logits(wfmt, W, L, D, X, B, js, -1, Zs, 1) == ORC_EINVAL);
  free(W); free(W2); free(Wu); free(Wr);
}

/* MX-scaled FP4: codecs, a block with a NaN, and a tiny step with its sampled entry points */
static void mxfp4(void) {
  for (int c = 0; c < 16; ++c) CHECK(fabs(orc_e2m1_value((uint8_t)c)) <= 6.0);
  CHECK(isnan(orc_e8m0_value(255)) && orc_e8m0_value(127) == 1.0);
  CHECK(orc_sr_e2m1(7.5, 3) == 7 && orc_sr_e2m1(-0.25, 65535) == 9);
  float t[32];
  uint32_t r[32];
  uint8_t codes[32], scale;
  for (int k = 0; k < 32; ++k) { t[k] = (float)(0.03 * rnd_gauss()); r[k] = rnd32() & 0xFFFF; }
  orc_mx_quantize_block(t, r, codes, &scale);
  CHECK(scale < 255);
  t[3] = NAN;
  orc_mx_quantize_block(t, r, codes, &scale);
  CHECK(scale == 255);
  enum { B = 4, D = 64, L = 19 };
  const int64_t rb = orc_mx_row_bytes(D);
  uint8_t* W = malloc((size_t)(rb * L));
  uint8_t* W2 = malloc((size_t)(rb * L));
  for (int64_t i = 0; i < rb * L; ++i) W[i] = (uint8_t)rnd32();
  for (int j = 0; j < L; ++j)
    for (int b = 0; b < D / 32; ++b) W[j * rb + D / 2 + b] = (uint8_t)(118 + (rnd32() % 4));
  uint16_t X[B * D];
  for (int i = 0; i < B * D; ++i) X[i] = orc_bf16_rne((float)(0.3 * rnd_gauss()));
  int32_t row_ptr[B + 1] = {0, 2, 2, 4, 5};
  int32_t ids[5] = {3, 18, 0, 3, 7};
  float dX[B * D], T[L * D];
  uint16_t G[B * L];
  memcpy(W2, W, (size_t)(rb * L));
  CHECK(orc_step(ORC_W_MXFP4, W2, L, D, X, B, row_ptr, ids, 0.05f, 2, 1, dX, NULL, NULL, G, 2) == ORC_OK);
  uint8_t* Wu = malloc((size_t)(rb * L));
  CHECK(orc_update_from_g(ORC_W_MXFP4, W, L, D, X, B, G, 0.05f, 2, 1, Wu, T, 1) == ORC_OK);
  CHECK(memcmp(Wu, W2, (size_t)(rb * L)) == 0);
  int64_t js[2] = {0, 18};
  uint8_t Wr[2 * 64];
  CHECK(orc_update_rows(ORC_W_MXFP4, W, L, D, X, B, row_ptr, ids, 0.05f, 2, 1, js, 2, Wr, NULL, NULL, 1) == ORC_OK);
  CHECK(memcmp(Wr + rb, W2 + 18 * rb, (size_t)rb) == 0);
  int32_t idx[2 * 3];
  CHECK(orc_topk(ORC_W_MXFP4, W, L, D, X, 2, 3, idx, NULL, 1) == ORC_OK);
  CHECK(orc_step(ORC_W_MXFP4, W2, L, 48, X, B, row_ptr, ids, 0.05f, 2, 1, dX, NULL, NULL, NULL, 1) == ORC_EINVAL);
  free(W); free(W2); free(Wu);
}

static void exact_and_kahan(void) {
  enum { B = 3, D = 5, L = 4 };
  double W[L * D], X[B * D], Y[B * L], Z[B * L], G[B * L], dX[B * D], dW[L * D], loss;
  for (int i = 0; i < L * D; ++i) W[i] = rnd_gauss();
  for (int i = 0; i < B * D; ++i) X[i] = rnd_gauss();
  for (int i = 0; i < B * L; ++i) Y[i] = (rnd32() & 3) == 0;
  CHECK(orc_grad_exact(L, D, B, W, X, Y, Z, G, dX, dW, &loss) == ORC_OK);
  CHECK(orc_grad_exact(L, D, B, W, X, Y, NULL, NULL, NULL, NULL, NULL) == ORC_OK);
  uint16_t w[9], c[9];
  float g[9];
  for (int i = 0; i < 9; ++i) { w[i] = orc_bf16_rne(1.0f); c[i] = 0; g[i] = (float)rnd_gauss(); }
  orc_kahan_update(9, w, c, g, 1e-3f);
  orc_kahan_update(0, w, c, g, 1e-3f);
}

int main(void) {
  codecs();
  rounding();
  step(ORC_W_BF16);
  step(ORC_W_E4M3);
  mxfp4();
  exact_and_kahan();
  printf("oracle sanitizer run: ok\n");
  return 0;
}
