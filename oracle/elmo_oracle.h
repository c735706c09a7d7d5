/*
 * CPU oracle for the ELMO classifier-head training step and top-k scoring.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The product path (the HIP library) never calls it, shares no code with
 * it, and fails loudly when its own extension is missing.
 *
 * What it computes (sources: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large
 * Output Spaces", atlas.scime.ai summary page, sections "Approach" and "Surprising findings"; the
 * arXiv abstract page of 2510.11168):
 *   - the classifier is trained in pure BF16 or FP8 E4M3 with no FP32 master weights and no tensor
 *     scaling, with stochastic rounding of the classifier update and plain momentum-free SGD;
 *   - the weight gradient is fused with the SGD update and the label dimension is chunked. Chunking
 *     and fusion only change where intermediates live, so this oracle computes the unchunked,
 *     unfused definition;
 *   - the loss is one-vs-all sigmoid binary cross-entropy, summed over samples and labels
 *     (the pages do not print it; this is the reading documented with the build).
 * Every floating-point quantisation point of the method is reproduced exactly; all sums run in
 * binary64 and are rounded once to binary32 where the method holds an FP32 value.
 *
 * All pointers are HOST pointers. Functions return 0 on success or a negative ORC_E* code.
 * Weight codes: BF16 as uint16 [L][D] row-major; E4M3 (OCP E4M3FN) as uint8 [L][D] row-major;
 * MXFP4 as rows of orc_mx_row_bytes(D) = D/2 + D/32 bytes: the E2M1 codes two per byte (element 2i in
 * the low nibble of byte i) then one E8M0 scale byte per 32-element block. For MXFP4, D % 32 == 0
 * and the forward operand is E4M3-RNE(X), as for E4M3 weights.
 * X: BF16 codes [B][D] row-major. Labels: CSR row_ptr[B+1], ids[row_ptr[B]], int32, set semantics.
 */
#ifndef ELMO_ORACLE_H
#define ELMO_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };
enum { ORC_W_BF16 = 0, ORC_W_E4M3 = 1, ORC_W_MXFP4 = 2 };

/* codecs */
double   orc_bf16_value(uint16_t code);
uint16_t orc_bf16_rne(float x);
double   orc_e4m3_value(uint8_t code);
uint8_t  orc_e4m3_rne_sat(double x);
/* stochastic rounding of an FP32 value with a 16-bit random integer r in [0, 65536) */
uint16_t orc_sr_bf16(float t, uint32_t r);
uint8_t  orc_sr_e4m3(float t, uint32_t r);
/* OCP MX FP4: E2M1 element (4-bit code) and E8M0 scale values; stochastic rounding of v (the value
 * already divided by the block's scale) to an E2M1 code with 16 random bits, saturating at 6; the
 * block exponent X = clamp(floor(log2 amax) - 2, -127, 127) (0 -> -127, inf -> 127, NaN -> 128);
 * one 32-element block: codes[k] (one per byte) and the scale code X + 127 (255 for a NaN block). */
double   orc_e2m1_value(uint8_t code);
double   orc_e8m0_value(uint8_t code);
uint8_t  orc_sr_e2m1(double v, uint32_t r);
int      orc_mx_block_exponent(float amax);
void     orc_mx_quantize_block(const float* t, const uint32_t* r, uint8_t* codes, uint8_t* scale);
int64_t  orc_mx_row_bytes(int D);
/* Philox4x32 (Salmon, Moraes, Dror, Shaw, SC'11) with the given number of rounds */
void     orc_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int rounds, uint32_t out[4]);
/* the 16 random bits used for weight element idx = j*D + k at (seed, step) */
uint32_t orc_r16(uint64_t seed, uint64_t step, uint64_t idx);
/* the sigmoid-BCE gradient code for logit z and label y (0 or 1): BF16-RNE of FP32(sigmoid(z) - y) */
uint16_t orc_grad_code(float z, int y);

/* array helpers (elementwise loops over the scalar functions above) */
void orc_bf16_rne_array(const float* x, uint16_t* out, int64_t n);
void orc_e4m3_rne_sat_array(const double* x, uint8_t* out, int64_t n);
void orc_sr_bf16_array(const float* t, const uint32_t* r, uint16_t* out, int64_t n);
void orc_sr_e4m3_array(const float* t, const uint32_t* r, uint8_t* out, int64_t n);
void orc_r16_array(uint64_t seed, uint64_t step, uint64_t idx0, uint32_t* out, int64_t n);

/* One full training step, in place on W. dX [B][D] is overwritten. Z ([B][L] FP32 logits) and
 * G ([B][L] BF16 gradient codes) are optional outputs (NULL to skip). loss (optional) receives the
 * summed BCE computed in binary64 from the FP32 logits. nthreads <= 0 uses the OpenMP default. */
int orc_step(int wfmt, void* W, int64_t L, int D, const uint16_t* X, int B,
             const int32_t* row_ptr, const int32_t* ids, float lr, uint64_t seed, uint64_t step,
             float* dX, double* loss, float* Z, uint16_t* G, int nthreads);

/* The weight half of the step given the gradient codes G ([B][L] BF16): dW = FP32(G^T X) with the
 * BF16 X, t = fmaf(-lr, dW, w), W_out = SR(t). W is not modified; Wout receives [L][D] codes and
 * Tout (nullable) the FP32 values t [L][D] before rounding. orc_step's weights equal this function
 * applied to orc_step's own G. */
int orc_update_from_g(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                      const uint16_t* G, float lr, uint64_t seed, uint64_t step, void* Wout, float* Tout,
                      int nthreads);

/* Sampled outputs of the same step for large shapes, without modifying W:
 *   orc_logits:      Z[b][i] for labels js[i] (all b)                      -> Z [B][nj]
 *   orc_update_rows: the updated codes of weight rows js[i]                 -> Wrows [nj][D]
 *                    (nullable: their gradient codes -> Grows [B][nj], and the FP32 values t
 *                    before rounding -> Trows [nj][D])
 *   orc_dx_rows:     dX rows bs[i] (sums over all L labels, pre-update W)  -> dXrows [nb][D] */
int orc_logits(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
               const int64_t* js, int nj, float* Z, int nthreads);
int orc_update_rows(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                    const int32_t* row_ptr, const int32_t* ids, float lr, uint64_t seed,
                    uint64_t step, const int64_t* js, int nj, void* Wrows, uint16_t* Grows,
                    float* Trows, int nthreads);
/* orc_update_rows with given gradient codes: G [B][nj] BF16 codes of labels js (teacher forcing). */
int orc_update_rows_from_g(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                           const uint16_t* G, float lr, uint64_t seed, uint64_t step, const int64_t* js,
                           int nj, void* Wrows, int nthreads);
int orc_dx_rows(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int B,
                const int32_t* row_ptr, const int32_t* ids, const int32_t* bs, int nb,
                float* dXrows, int nthreads);

/* Unquantised binary64 reference of the same loss and gradients (for finite-difference checks).
 * Y is dense [B][L] with entries 0/1. Any output pointer may be NULL. */
int orc_grad_exact(int64_t L, int D, int B, const double* W, const double* X, const double* Y,
                   double* Z, double* G, double* dX, double* dW, double* loss);

/* Top-k scoring: score[n][j] = FP32(sum_k xt[n][k] * w[j][k]) with xt = X (BF16 weights) or
 * E4M3-RNE(X) (E4M3 weights); rows ranked by (score desc, label asc), NaN after every number.
 * idx [N][k] int32, score [N][k] FP32 (score may be NULL). */
int orc_topk(int wfmt, const void* W, int64_t L, int D, const uint16_t* X, int N, int k,
             int32_t* idx, float* score, int nthreads);

/* Kahan-compensated BF16 update of n encoder parameters, in place: parameter w[i] and its
 * compensation c[i] BF16, gradient g[i] and lr binary32 (reading of "Kahan summation (encoder)",
 * ELMO summary, Approach). Per element, in binary32, both stores rounded to BF16 by RNE:
 *   d = -lr g;  y = d - c;  t = bf16(w + y);  c' = bf16((t - w) - y);  w' = t.  */
void orc_kahan_update(int64_t n, uint16_t* w, uint16_t* c, const float* g, float lr);

#ifdef __cplusplus
}
#endif
#endif
