/*
 * CPU oracle for the ELMO classifier-head step — TEST INFRASTRUCTURE ONLY (see elmo_oracle.h).
 *
 * Plain C, binary64 accumulation, OpenMP over independent outputs only. It follows the method as
 * the ELMO pages describe it ("ELMO: Efficiency via Low-precision and Peak Memory Optimization in
 * Large Output Spaces": atlas.scime.ai summary, sections "Approach" and "Surprising findings";
 * arXiv 2510.11168 abstract): pure BF16 / FP8-E4M3 classifier weights, no master weights, no
 * tensor scaling, stochastic rounding of the update, momentum-free SGD. Where the pages are silent
 * (loss, RNG, rounding of intermediates) the documented readings are implemented and named below.
 *
 * Shares no code with the HIP library; written independently from the definitions.
 */
#include "elmo_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------------
 * BF16: a BF16 value is the binary32 value whose upper 16 bits are the code and lower 16 bits are 0.
 * ---------------------------------------------------------------------------------------------- */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

double orc_bf16_value(uint16_t code) { return (double)f32_from_bits((uint32_t)code << 16); }

/* Distance from a BF16 magnitude pattern (upper 16 bits of a binary32 magnitude) to the next one up,
 * as a binary64 number: one unit in the last of its 8 significand bits. */
static double bf16_ulp_above(uint32_t mag_bits) {
  int e = (int)(mag_bits >> 23);            /* biased binary32 exponent */
  if (e == 0) e = 1;                        /* subnormals share the spacing of the smallest normal */
  return ldexp(1.0, e - 127 - 7);
}

/* Round-to-nearest-even from binary32 to BF16, decided by comparing distances to the two
 * neighbouring BF16 values. Overflow goes to infinity as in IEEE 754. NaN stays a quiet NaN. */
uint16_t orc_bf16_rne(float x) {
  uint32_t u = bits_from_f32(x);
  uint32_t s = u & 0x80000000u, a = u & 0x7fffffffu;
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lo = a & 0xffff0000u;            /* largest BF16 magnitude <= |x| */
  if (lo == a) return (uint16_t)((s | a) >> 16);
  double dlo = (double)f32_from_bits(lo);
  double dhi = dlo + bf16_ulp_above(lo);    /* next BF16 magnitude (2^128 stands for infinity) */
  double da = (double)fabsf(x);
  double el = da - dlo, eh = dhi - da;
  uint32_t pick;
  if (el < eh) pick = lo;
  else if (eh < el) pick = lo + 0x10000u;
  else pick = ((lo >> 16) & 1u) ? lo + 0x10000u : lo;   /* tie: even last significand bit */
  return (uint16_t)((s | pick) >> 16);
}

/* ------------------------------------------------------------------------------------------------
 * OCP FP8 E4M3 ("E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal; S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
 * ---------------------------------------------------------------------------------------------- */
double orc_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Largest code c in [0, 0x7E] with value(c) <= a, for 0 <= a < 448 (codes ascend with value). */
static int e4m3_floor_code(double a) {
  int lo = 0, hi = 0x7E;                    /* invariant: value(lo) <= a < value(hi + 1) */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (orc_e4m3_value((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* Round-to-nearest-even with saturation to the largest finite magnitude (448). */
uint8_t orc_e4m3_rne_sat(double x) {
  uint8_t s = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(s | 0x7F);
  double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(s | 0x7E);
  int c = e4m3_floor_code(a);
  double lo = orc_e4m3_value((uint8_t)c);
  if (lo == a) return (uint8_t)(s | c);
  double hi = orc_e4m3_value((uint8_t)(c + 1));
  double el = a - lo, eh = hi - a;
  int pick = (el < eh) ? c : (eh < el) ? c + 1 : ((c & 1) ? c + 1 : c);  /* tie: even mantissa */
  return (uint8_t)(s | pick);
}

/* ------------------------------------------------------------------------------------------------
 * Stochastic rounding (the pages name "stochastic rounding (classifier)" but not its mechanism).
 * Reading: with a = |t|, lo the largest format value <= a, u the spacing above lo and
 * q = floor((a - lo) / u * 2^16), round the magnitude up to lo + u iff q + r >= 2^16, where r is a
 * uniform 16-bit integer; then reapply the sign. E4M3 saturates at 448; NaN stays NaN.
 * ---------------------------------------------------------------------------------------------- */
uint16_t orc_sr_bf16(float t, uint32_t r) {
  if (isnan(t)) return orc_bf16_rne(t);
  uint32_t u = bits_from_f32(t);
  uint32_t s = u & 0x80000000u, a = u & 0x7fffffffu;
  if (isinf(t)) return (uint16_t)((s | a) >> 16);
  uint32_t lo = a & 0xffff0000u;
  if (lo == a) return (uint16_t)((s | a) >> 16);
  double ulp = bf16_ulp_above(lo);
  double q = floor(((double)f32_from_bits(a) - (double)f32_from_bits(lo)) / ulp * 65536.0);
  uint32_t pick = ((uint32_t)q + (r & 0xFFFFu) >= 65536u) ? lo + 0x10000u : lo;
  return (uint16_t)((s | pick) >> 16);
}

uint8_t orc_sr_e4m3(float t, uint32_t r) {
  uint8_t s = signbit(t) ? 0x80 : 0x00;
  if (isnan(t)) return (uint8_t)(s | 0x7F);
  double a = fabs((double)t);
  if (a >= 448.0) return (uint8_t)(s | 0x7E);
  int c = e4m3_floor_code(a);
  double lo = orc_e4m3_value((uint8_t)c);
  if (lo == a) return (uint8_t)(s | c);
  double u = orc_e4m3_value((uint8_t)(c + 1)) - lo;
  double q = floor((a - lo) / u * 65536.0);
  int pick = ((uint32_t)q + (r & 0xFFFFu) >= 65536u) ? c + 1 : c;
  return (uint8_t)(s | pick);
}

/* ------------------------------------------------------------------------------------------------
 * MX-scaled FP4 (OCP Microscaling formats): blocks of 32 E2M1 elements sharing one E8M0 scale.
 * E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal (m x 0.5); no
 * infinity or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. E8M0: the power of two 2^(c - 127),
 * c = 255 is NaN. The pages name FP4 weights as the recipe gap that needs micro-tensor scaling
 * (summary page, Limitations); the scaling rule and the rounding of the elements are the reading
 * documented with the build: the block's shared exponent is floor(log2(max |t|)) minus the element
 * format's largest exponent (2), clamped to the scale's range; each element t / 2^X is rounded to
 * E2M1 stochastically with the rule of orc_sr_bf16 (16 random bits), saturating at 6.
 * ---------------------------------------------------------------------------------------------- */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint8_t code) {
  double v = e2m1_mag[code & 7];
  return (code & 8) ? -v : v;
}

double orc_e8m0_value(uint8_t code) { return code == 255 ? NAN : ldexp(1.0, (int)code - 127); }

uint8_t orc_sr_e2m1(double v, uint32_t r) {
  uint8_t s = signbit(v) ? 8 : 0;
  double a = fabs(v);
  if (a >= 6.0) return (uint8_t)(s | 7);
  int c = 0;
  while (c < 7 && e2m1_mag[c + 1] <= a) c++;        /* largest magnitude <= a */
  if (e2m1_mag[c] == a) return (uint8_t)(s | c);
  double u = e2m1_mag[c + 1] - e2m1_mag[c];
  double q = floor((a - e2m1_mag[c]) / u * 65536.0);
  return (uint8_t)(s | (((uint32_t)q + (r & 0xFFFFu) >= 65536u) ? c + 1 : c));
}

int orc_mx_block_exponent(float amax) {
  if (isnan(amax)) return 128;                       /* marks a NaN block (scale code 255) */
  if (amax == 0.0f) return -127;
  if (isinf(amax)) return 127;
  int x = ilogb((double)amax) - 2;                   /* floor(log2 amax) - (largest E2M1 exponent) */
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

void orc_mx_quantize_block(const float* t, const uint32_t* r, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  int nan = 0;
  for (int k = 0; k < 32; k++) {
    if (isnan(t[k])) nan = 1;
    else if (fabsf(t[k]) > amax) amax = fabsf(t[k]);
  }
  int x = nan ? 128 : orc_mx_block_exponent(amax);
  if (x == 128) {
    *scale = 255;
    for (int k = 0; k < 32; k++) codes[k] = 0;
    return;
  }
  *scale = (uint8_t)(x + 127);
  for (int k = 0; k < 32; k++) codes[k] = orc_sr_e2m1(ldexp((double)t[k], -x), r[k]);
}

/* ------------------------------------------------------------------------------------------------
 * Philox4x32 as defined in "Parallel Random Numbers: As Easy as 1, 2, 3" (Salmon et al., SC'11):
 * each round multiplies counter words 0 and 2 by two fixed 32-bit constants, and the new counter
 * is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key is advanced by the
 * Weyl constants between rounds.
 * ---------------------------------------------------------------------------------------------- */
void orc_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds, uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int i = 0; i < rounds; i++) {
    if (i > 0) { k0 += W0; k1 += W1; }
    uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* RNG keying (reading of "counter-based, keyed on seed, step and element index"): key = seed,
 * counter = (g, step) as 64-bit halves, ten rounds; the 128 output bits give 16 bits to each of 8
 * elements. The 8 consecutive element indices 8g .. 8g + 7 share block g = idx >> 3; the element at
 * position p = idx & 7 takes 16-bit half (p & 1) of output word p >> 1. The index idx = j*D + k runs
 * over the whole weight matrix, so the draw of an element does not depend on how the labels are
 * chunked or tiled. */
uint32_t orc_r16(uint64_t seed, uint64_t step, uint64_t idx) {
  uint64_t g = idx >> 3;
  unsigned p = (unsigned)(idx & 7);
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t x[4];
  orc_philox4x32(ctr, key, 10, x);
  uint32_t word = x[p >> 1];
  return (word >> (16 * (p & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------------------------------
 * Sigmoid-BCE gradient. g = sigmoid(z) - y, evaluated in binary64 in the algebraically equal forms
 * 1/(1+e^-z) (y = 0) and -1/(1+e^z) (y = 1), then rounded to binary32 (the precision in which a
 * device holds g) and from there to BF16 with round-to-nearest-even.
 * ---------------------------------------------------------------------------------------------- */
static double grad64(double z, int y) {
  return y ? -1.0 / (1.0 + exp(z)) : 1.0 / (1.0 + exp(-z));
}

uint16_t orc_grad_code(float z, int y) { return orc_bf16_rne((float)grad64((double)z, y)); }

static double bce64(double z, int y) {
  return (z > 0.0 ? z : 0.0) - (y ? z : 0.0) + log1p(exp(-fabs(z)));
}

/* ------------------------------------------------------------------------------------------------
 * array helpers
 * ---------------------------------------------------------------------------------------------- */
void orc_bf16_rne_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_rne(x[i]);
}
void orc_e4m3_rne_sat_array(const double* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_rne_sat(x[i]);
}
void orc_sr_bf16_array(const float* t, const uint32_t* r, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_sr_bf16(t[i], r[i]);
}
void orc_sr_e4m3_array(const float* t, const uint32_t* r, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_sr_e4m3(t[i], r[i]);
}
void orc_r16_array(uint64_t seed, uint64_t step, uint64_t idx0, uint32_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_r16(seed, step, idx0 + (uint64_t)i);
}

/* ------------------------------------------------------------------------------------------------
 * the training step
 * ---------------------------------------------------------------------------------------------- */
static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* decoded value of weight element (j, k) */
/* MXFP4 rows: D / 2 bytes of E2M1 codes (element 2i in the low nibble of byte i, 2i + 1 in the high
 * nibble), then D / 32 E8M0 scale bytes (block b = elements 32b .. 32b + 31) */
int64_t orc_mx_row_bytes(int D) { return (int64_t)D / 2 + D / 32; }

static double wval(int wfmt, const void* W, int64_t j, int D, int k) {
  if (wfmt == ORC_W_MXFP4) {
    const uint8_t* row = (const uint8_t*)W + j * orc_mx_row_bytes(D);
    uint8_t byte = row[k / 2];
    return orc_e2m1_value((uint8_t)((k & 1) ? byte >> 4 : byte & 15)) * orc_e8m0_value(row[D / 2 + k / 32]);
  }
  int64_t i = j * (int64_t)D + k;
  return wfmt == ORC_W_BF16 ? orc_bf16_value(((const uint16_t*)W)[i])
                            : orc_e4m3_value(((const uint8_t*)W)[i]);
}

/* the updated codes of weight row j from its FP32 values t[0..D): per element for BF16 and E4M3;
 * per 32-element block for MXFP4. The row is written at row `i` of Wout. */
static void write_row(int wfmt, void* Wout, int64_t i, int64_t j, int D, const float* t, uint64_t seed,
                      uint64_t step) {
  if (wfmt == ORC_W_MXFP4) {
    uint8_t* row = (uint8_t*)Wout + i * orc_mx_row_bytes(D);
    for (int b = 0; b < D / 32; b++) {
      uint32_t r[32];
      uint8_t codes[32];
      for (int k = 0; k < 32; k++) r[k] = orc_r16(seed, step, (uint64_t)(j * (int64_t)D + 32 * b + k));
      orc_mx_quantize_block(t + 32 * b, r, codes, &row[D / 2 + b]);
      for (int k = 0; k < 32; k += 2) row[(32 * b + k) / 2] = (uint8_t)(codes[k] | (codes[k + 1] << 4));
    }
    return;
  }
  for (int k = 0; k < D; k++) {
    int64_t o = i * (int64_t)D + k;
    uint32_t r = orc_r16(seed, step, (uint64_t)(j * (int64_t)D + k));
    if (wfmt == ORC_W_BF16) ((uint16_t*)Wout)[o] = orc_sr_bf16(t[k], r);
    else ((uint8_t*)Wout)[o] = orc_sr_e4m3(t[k], r);
  }
}

/* per-sample label sets, sorted and deduplicated, for membership tests */
typedef struct { int32_t* v; int64_t* off; } labelsets;

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static int labelsets_build(labelsets* s, int B, int64_t L, const int32_t* row_ptr, const int32_t* ids) {
  int64_t nnz = row_ptr[B];
  s->v = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  s->off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B + 1));
  if (!s->v || !s->off) { free(s->v); free(s->off); return ORC_ENOMEM; }
  int64_t w = 0;
  for (int b = 0; b < B; b++) {
    s->off[b] = w;
    int64_t r0 = row_ptr[b], r1 = row_ptr[b + 1];
    if (r1 < r0) { free(s->v); free(s->off); return ORC_EINVAL; }
    int64_t start = w;
    for (int64_t i = r0; i < r1; i++) {
      if (ids[i] < 0 || ids[i] >= L) { free(s->v); free(s->off); return ORC_EINVAL; }
      s->v[w++] = ids[i];
    }
    qsort(s->v + start, (size_t)(w - start), sizeof(int32_t), cmp_i32);
    int64_t u = start;                      /* drop duplicates: the labels are a set */
    for (int64_t i = start; i < w; i++)
      if (i == start || s->v[i] != s->v[i - 1]) s->v[u++] = s->v[i];
    w = u;
  }
  s->off[B] = w;
  return ORC_OK;
}

static void labelsets_free(labelsets* s) { free(s->v); free(s->off); }

static int has_label(const labelsets* s, int b, int64_t j) {
  int32_t key = (int32_t)j;
  return bsearch(&key, s->v + s->off[b], (size_t)(s->off[b + 1] - s->off[b]), sizeof(int32_t),
                 cmp_i32) != NULL;
}

/* X as used by the forward contraction: X itself for BF16 weights, E4M3-RNE(X) for E4M3 weights
 * (configuration text: "X cast to E4M3 for the forward MFMA"). */
static double* forward_x(int wfmt, const uint16_t* X, int B, int D) {
  double* xt = (double*)malloc(sizeof(double) * (size_t)B * D);
  if (!xt) return NULL;
  for (int64_t i = 0; i < (int64_t)B * D; i++) {
    double v = orc_bf16_value(X[i]);
    xt[i] = wfmt == ORC_W_BF16 ? v : orc_e4m3_value(orc_e4m3_rne_sat(v));   /* E4M3 and MXFP4 */
  }
  return xt;
}

static double* backward_x(const uint16_t* X, int B, int D) {
  double* xb = (double*)malloc(sizeof(double) * (size_t)B * D);
  if (!xb) return NULL;
  for (int64_t i = 0; i < (int64_t)B * D; i++) xb[i] = orc_bf16_value(X[i]);
  return xb;
}

/* z_bj = FP32(sum_k xt_bk * w_jk); every product is exact in binary64 */
static float logit(int wfmt, const void* W, int64_t j, int D, const double* xt_row) {
  double s = 0.0;
  for (int k = 0; k < D; k++) s += xt_row[k] * wval(wfmt, W, j, D, k);
  return (float)s;
}

/* SGD without momentum: t = fmaf(-lr, dW, w), one FP32 rounding */
static float sgd_t(double w, float dw, float lr) { return fmaf(-lr, dw, (float)w); }

static int check_common(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B) {
  if (wfmt != ORC_W_BF16 && wfmt != ORC_W_E4M3 && wfmt != ORC_W_MXFP4) return ORC_EINVAL;
  if (wfmt == ORC_W_MXFP4 && (D % 32 != 0 || D > 4096)) return ORC_EINVAL;
  if (!W || !X || L < 1 || D < 1 || B < 1) return ORC_EINVAL;
  return ORC_OK;
}

int orc_step(int wfmt, void* W, int64_t L, int D, const uint16_t* X, int B,
             const int32_t* row_ptr, const int32_t* ids, float lr, uint64_t seed, uint64_t step,
             float* dX, double* loss, float* Zout, uint16_t* Gout, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!row_ptr || (!ids && row_ptr[B] > 0) || !dX) return ORC_EINVAL;
  set_threads(nthreads);
  labelsets ls;
  if ((rc = labelsets_build(&ls, B, L, row_ptr, ids))) return rc;
  double* xt = forward_x(wfmt, X, B, D);
  double* xb = backward_x(X, B, D);
  uint16_t* G = Gout ? Gout : (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * (size_t)L);
  if (!xt || !xb || !G) { free(xt); free(xb); if (!Gout) free(G); labelsets_free(&ls); return ORC_ENOMEM; }
  double lsum = 0.0;

  /* forward contraction, gradient and (optionally) loss, per label */
  #pragma omp parallel for schedule(static) reduction(+ : lsum)
  for (int64_t j = 0; j < L; j++) {
    for (int b = 0; b < B; b++) {
      float z = logit(wfmt, W, j, D, xt + (int64_t)b * D);
      int y = has_label(&ls, b, j);
      G[(int64_t)b * L + j] = orc_grad_code(z, y);
      if (Zout) Zout[(int64_t)b * L + j] = z;
      if (loss) lsum += bce64((double)z, y);
    }
  }

  /* input gradient with the pre-update weights: dX_bk = FP32(sum_j g_bj * w_jk) */
  #pragma omp parallel for schedule(static)
  for (int b = 0; b < B; b++) {
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    for (int64_t j = 0; j < L; j++) {
      double g = orc_bf16_value(G[(int64_t)b * L + j]);
      for (int k = 0; k < D; k++) acc[k] += g * wval(wfmt, W, j, D, k);
    }
    for (int k = 0; k < D; k++) dX[(int64_t)b * D + k] = (float)acc[k];
    free(acc);
  }

  /* weight gradient dW_jk = FP32(sum_b g_bj * x_bk) with the BF16 X, then SGD + SR in place (the
   * whole row's t first: an MXFP4 block shares its scale) */
  #pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < L; j++) {
    float t[4096];
    for (int k = 0; k < D; k++) {
      double s = 0.0;
      for (int b = 0; b < B; b++) s += orc_bf16_value(G[(int64_t)b * L + j]) * xb[(int64_t)b * D + k];
      t[k] = sgd_t(wval(wfmt, W, j, D, k), (float)s, lr);
    }
    write_row(wfmt, W, j, j, D, t, seed, step);
  }

  if (loss) *loss = lsum;
  if (!Gout) free(G);
  free(xt); free(xb); labelsets_free(&ls);
  return ORC_OK;
}

int orc_update_from_g(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                      const uint16_t* G, float lr, uint64_t seed, uint64_t step, void* Wout, float* Tout,
                      int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!G || !Wout) return ORC_EINVAL;
  set_threads(nthreads);
  double* xb = backward_x(X, B, D);
  if (!xb) return ORC_ENOMEM;
  #pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < L; j++) {
    float t[4096];
    for (int k = 0; k < D; k++) {
      double s = 0.0;
      for (int b = 0; b < B; b++) s += orc_bf16_value(G[(int64_t)b * L + j]) * xb[(int64_t)b * D + k];
      t[k] = sgd_t(wval(wfmt, W, j, D, k), (float)s, lr);
      if (Tout) Tout[j * (int64_t)D + k] = t[k];
    }
    write_row(wfmt, Wout, j, j, D, t, seed, step);
  }
  free(xb);
  return ORC_OK;
}

int orc_logits(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
               const int64_t* js, int nj, float* Z, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!js || !Z || nj < 0) return ORC_EINVAL;
  for (int i = 0; i < nj; i++) if (js[i] < 0 || js[i] >= L) return ORC_EINVAL;
  set_threads(nthreads);
  double* xt = forward_x(wfmt, X, B, D);
  if (!xt) return ORC_ENOMEM;
  #pragma omp parallel for schedule(static)
  for (int i = 0; i < nj; i++)
    for (int b = 0; b < B; b++) Z[(int64_t)b * nj + i] = logit(wfmt, W, js[i], D, xt + (int64_t)b * D);
  free(xt);
  return ORC_OK;
}

/* Row j's update given its gradient values g[b] (BF16 values): dW_jk = FP32(sum_b g_b x_bk), summed
 * in binary64 over b ascending; t = fmaf(-lr, dW, w); SR with the draw of element j*D + k; output
 * row i of Wrows (and of Trows, the FP32 t, when not NULL). */
static void update_row(int wfmt, const void* W, int64_t j, int D, const double* xb, const double* g, int B,
                       float lr, uint64_t seed, uint64_t step, void* Wrows, float* Trows, int i) {
  float t[4096];
  for (int k = 0; k < D; k++) {
    double s = 0.0;
    for (int b = 0; b < B; b++) s += g[b] * xb[(int64_t)b * D + k];
    t[k] = sgd_t(wval(wfmt, W, j, D, k), (float)s, lr);
    if (Trows) Trows[(int64_t)i * D + k] = t[k];
  }
  write_row(wfmt, Wrows, i, j, D, t, seed, step);
}

int orc_update_rows(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                    const int32_t* row_ptr, const int32_t* ids, float lr, uint64_t seed,
                    uint64_t step, const int64_t* js, int nj, void* Wrows, uint16_t* Grows,
                    float* Trows, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!row_ptr || (!ids && row_ptr[B] > 0) || !js || !Wrows || nj < 0) return ORC_EINVAL;
  for (int i = 0; i < nj; i++) if (js[i] < 0 || js[i] >= L) return ORC_EINVAL;
  set_threads(nthreads);
  labelsets ls;
  if ((rc = labelsets_build(&ls, B, L, row_ptr, ids))) return rc;
  double* xt = forward_x(wfmt, X, B, D);
  double* xb = backward_x(X, B, D);
  if (!xt || !xb) { free(xt); free(xb); labelsets_free(&ls); return ORC_ENOMEM; }
  #pragma omp parallel for schedule(static)
  for (int i = 0; i < nj; i++) {
    int64_t j = js[i];
    double* g = (double*)malloc(sizeof(double) * (size_t)B);
    for (int b = 0; b < B; b++) {
      uint16_t gc = orc_grad_code(logit(wfmt, W, j, D, xt + (int64_t)b * D), has_label(&ls, b, j));
      if (Grows) Grows[(int64_t)b * nj + i] = gc;
      g[b] = orc_bf16_value(gc);
    }
    update_row(wfmt, W, j, D, xb, g, B, lr, seed, step, Wrows, Trows, i);
    free(g);
  }
  free(xt); free(xb); labelsets_free(&ls);
  return ORC_OK;
}

int orc_update_rows_from_g(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                           const uint16_t* G, float lr, uint64_t seed, uint64_t step, const int64_t* js,
                           int nj, void* Wrows, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!G || !js || !Wrows || nj < 0) return ORC_EINVAL;
  for (int i = 0; i < nj; i++) if (js[i] < 0 || js[i] >= L) return ORC_EINVAL;
  set_threads(nthreads);
  double* xb = backward_x(X, B, D);
  if (!xb) return ORC_ENOMEM;
  #pragma omp parallel for schedule(static)
  for (int i = 0; i < nj; i++) {
    double* g = (double*)malloc(sizeof(double) * (size_t)B);
    for (int b = 0; b < B; b++) g[b] = orc_bf16_value(G[(int64_t)b * nj + i]);
    update_row(wfmt, W, js[i], D, xb, g, B, lr, seed, step, Wrows, NULL, i);
    free(g);
  }
  free(xb);
  return ORC_OK;
}

int orc_dx_rows(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                const int32_t* row_ptr, const int32_t* ids, const int32_t* bs, int nb,
                float* dXrows, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, B);
  if (rc) return rc;
  if (!row_ptr || (!ids && row_ptr[B] > 0) || !bs || !dXrows || nb < 0) return ORC_EINVAL;
  for (int i = 0; i < nb; i++) if (bs[i] < 0 || bs[i] >= B) return ORC_EINVAL;
  set_threads(nthreads);
  labelsets ls;
  if ((rc = labelsets_build(&ls, B, L, row_ptr, ids))) return rc;
  double* xt = forward_x(wfmt, X, B, D);
  if (!xt) { labelsets_free(&ls); return ORC_ENOMEM; }
  for (int i = 0; i < nb; i++) {
    int b = bs[i];
    int nt = 1;
#ifdef _OPENMP
    nt = omp_get_max_threads();
#endif
    /* per-thread partial sums over contiguous label ranges, added in thread order */
    double* part = (double*)calloc((size_t)nt * D, sizeof(double));
    #pragma omp parallel num_threads(nt)
    {
      int t = 0;
#ifdef _OPENMP
      t = omp_get_thread_num();
#endif
      double* acc = part + (int64_t)t * D;
      int64_t j0 = L * t / nt, j1 = L * (t + 1) / nt;
      for (int64_t j = j0; j < j1; j++) {
        double g = orc_bf16_value(orc_grad_code(logit(wfmt, W, j, D, xt + (int64_t)b * D), has_label(&ls, b, j)));
        for (int k = 0; k < D; k++) acc[k] += g * wval(wfmt, W, j, D, k);
      }
    }
    for (int k = 0; k < D; k++) {
      double s = 0.0;
      for (int t = 0; t < nt; t++) s += part[(int64_t)t * D + k];
      dXrows[(int64_t)i * D + k] = (float)s;
    }
    free(part);
  }
  free(xt); labelsets_free(&ls);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * unquantised binary64 loss and gradients: Z = X W^T, L = sum BCE(Z, Y), G = dL/dZ = sigmoid(Z) - Y,
 * dX = G W, dW = G^T X.
 * ---------------------------------------------------------------------------------------------- */
int orc_grad_exact(int64_t L, int D, int B, const double* W, const double* X, const double* Y,
                   double* Z, double* G, double* dX, double* dW, double* loss) {
  if (!W || !X || !Y || L < 1 || D < 1 || B < 1) return ORC_EINVAL;
  double* z = (double*)malloc(sizeof(double) * (size_t)B * L);
  double* g = (double*)malloc(sizeof(double) * (size_t)B * L);
  if (!z || !g) { free(z); free(g); return ORC_ENOMEM; }
  double lsum = 0.0;
  for (int b = 0; b < B; b++)
    for (int64_t j = 0; j < L; j++) {
      double s = 0.0;
      for (int k = 0; k < D; k++) s += X[(int64_t)b * D + k] * W[j * D + k];
      int y = Y[(int64_t)b * L + j] != 0.0;
      z[(int64_t)b * L + j] = s;
      g[(int64_t)b * L + j] = grad64(s, y);
      lsum += bce64(s, y);
    }
  if (dX)
    for (int b = 0; b < B; b++)
      for (int k = 0; k < D; k++) {
        double s = 0.0;
        for (int64_t j = 0; j < L; j++) s += g[(int64_t)b * L + j] * W[j * D + k];
        dX[(int64_t)b * D + k] = s;
      }
  if (dW)
    for (int64_t j = 0; j < L; j++)
      for (int k = 0; k < D; k++) {
        double s = 0.0;
        for (int b = 0; b < B; b++) s += g[(int64_t)b * L + j] * X[(int64_t)b * D + k];
        dW[j * D + k] = s;
      }
  if (Z) memcpy(Z, z, sizeof(double) * (size_t)B * L);
  if (G) memcpy(G, g, sizeof(double) * (size_t)B * L);
  if (loss) *loss = lsum;
  free(z); free(g);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * top-k by (score desc, label asc), NaN scores after all numbers
 * ---------------------------------------------------------------------------------------------- */
static int ranks_before(float sa, int64_t ja, float sb, int64_t jb) {
  int na = isnan(sa), nb = isnan(sb);
  if (na != nb) return nb;                  /* a number ranks before NaN */
  if (!na && sa != sb) return sa > sb;
  return ja < jb;
}

int orc_topk(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int N, int k,
             int32_t* idx, float* score, int nthreads) {
  int rc = check_common(wfmt, W, L, D, X, N);
  if (rc) return rc;
  if (k < 1 || k > L || !idx) return ORC_EINVAL;
  set_threads(nthreads);
  double* xt = forward_x(wfmt, X, N, D);
  if (!xt) return ORC_ENOMEM;
  #pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < N; n++) {
    float* bs = (float*)malloc(sizeof(float) * (size_t)k);
    int64_t* bj = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
    int cnt = 0;
    for (int64_t j = 0; j < L; j++) {
      float s = logit(wfmt, W, j, D, xt + (int64_t)n * D);
      if (cnt == k && !ranks_before(s, j, bs[k - 1], bj[k - 1])) continue;
      int p = cnt < k ? cnt++ : k - 1;      /* insertion into the sorted best list */
      while (p > 0 && ranks_before(s, j, bs[p - 1], bj[p - 1])) { bs[p] = bs[p - 1]; bj[p] = bj[p - 1]; p--; }
      bs[p] = s; bj[p] = j;
    }
    for (int i = 0; i < k; i++) {
      idx[(int64_t)n * k + i] = (int32_t)bj[i];
      if (score) score[(int64_t)n * k + i] = bs[i];
    }
    free(bs); free(bj);
  }
  free(xt);
  return ORC_OK;
}

/* ------------------------------------------------------------------------------------------------
 * Kahan-compensated BF16 update (encoder parameters). The pages train the encoder with Kahan
 * summation and no FP32 master weights (ELMO summary, Approach); they fix neither the precision
 * of the compensation nor the order of operations. Reading: the compensation is a BF16 buffer
 * beside the BF16 parameters, and each step is one step of Kahan's compensated summation of the
 * increments d = -lr g, with w the running sum and c the negated low part it lost:
 *   y = d - c,  t = w + y (stored as BF16),  c = (t - w) - y (stored as BF16),  w = t,
 * evaluated in binary32 (t - w of two BF16 values is exact there).
 * ---------------------------------------------------------------------------------------------- */
void orc_kahan_update(int64_t n, uint16_t* w, uint16_t* c, const float* g, float lr) {
  for (int64_t i = 0; i < n; ++i) {
    const float wv = f32_from_bits((uint32_t)w[i] << 16);
    const float cv = f32_from_bits((uint32_t)c[i] << 16);
    const float d = -lr * g[i];
    const float y = d - cv;
    const uint16_t t = orc_bf16_rne(wv + y);
    const float tv = f32_from_bits((uint32_t)t << 16);
    c[i] = orc_bf16_rne((tv - wv) - y);
    w[i] = t;
  }
}
