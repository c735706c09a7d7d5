/*
 * elmo_xmc — MI355X (gfx950) library for the chunked, fused, low-precision training step of an
 * extreme-multilabel (XMC) linear classifier head, and its top-k scoring pass.
 *
 * Method: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large Output Spaces"
 * (atlas.scime.ai summary, sections "Approach" and "Surprising findings"; arXiv 2510.11168,
 * abstract). The classifier weights are stored in pure BF16 or FP8 E4M3 with no FP32 master copy
 * and no tensor scaling; the weight gradient is fused into a momentum-free SGD update that writes
 * the weights back in place with stochastic rounding; the label dimension is processed in chunks
 * so that transient memory is bounded by one chunk.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (allocated by the caller on the current HIP device) unless noted.
 *     The library never allocates or frees device memory and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is enqueued asynchronously on
 *     it; the call returns before the device finishes. Device-side faults surface at the caller's
 *     next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a negative elmo_status is
 *     returned and nothing runs. After each launch the HIP error state is checked (ELMO_EHIP).
 *   - Pointers must be 16-byte aligned. Buffers must not alias each other.
 *   - No C++ exception crosses this interface. Nothing is printed.
 */
#ifndef ELMO_XMC_H
#define ELMO_XMC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ELMO_OK = 0,
  ELMO_EINVAL = -1,        /* null pointer, misalignment, bad scalar argument            */
  ELMO_ESHAPE = -2,        /* B, D, L, N, k or chunk outside the supported ranges        */
  ELMO_EDTYPE = -3,        /* unknown weight format                                      */
  ELMO_EWORKSPACE = -4,    /* workspace missing or smaller than the *_workspace_bytes   */
  ELMO_EHIP = -5,          /* a HIP runtime call or kernel launch failed                 */
  ELMO_EUNSUPPORTED = -6,  /* valid request that this library does not implement         */
  ELMO_ESCRATCH = -7       /* step too large for elmo_xmc_step_noalloc's static scratch  */
} elmo_status;

/* Weight storage formats. BF16: uint16 codes. E4M3: OCP FP8 E4M3FN codes (uint8; max 448, no
 * infinity, 0x7F/0xFF NaN) — the "E4M3" of the summary page's "Surprising findings".
 * MXFP4: OCP Microscaling FP4 (the FP4 weights that the summary page's "Limitations" leave to
 * micro-tensor scaling): each row is D/2 bytes of E2M1 codes (element 2i in the low nibble of byte
 * i, 2i+1 in the high nibble; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) followed by D/32 E8M0 scale
 * bytes (2^(c-127), 255 = NaN), scale b applying to elements 32b .. 32b+31: 17*D/32 bytes per row,
 * "L x D" below meaning L such rows. Requires D % 256 == 0. The forward scores against
 * E4M3-RNE(X); the update recomputes each block's scale from the new values t: X = floor(log2
 * max|t|) - 2 clamped to [-127, 127] (an all-zero block takes -127, a block with a NaN scale 255
 * and zero codes), then each element SR(t / 2^X) to E2M1 with the element's 16 random bits (the
 * same rule and draws as the other formats), saturating at magnitude 6. */
enum { ELMO_W_BF16 = 0, ELMO_W_E4M3 = 1, ELMO_W_MXFP4 = 2 };

/* Supported shapes: 1 <= B <= 256; 64 <= D <= 1024 with D % 64 == 0 (MXFP4: D % 256 == 0); 1 <= L < 2^31;
 * chunk >= 1 (rounded down internally to a multiple of 128 labels, at least 128, and capped so that
 * one chunk of weight rows stays below 2 GiB). */
#define ELMO_MAX_B 256
#define ELMO_MAX_D 1024
#define ELMO_MAX_TOPK 64

int elmo_abi_version(void);
const char* elmo_status_str(int status);

/*
 * One training step of the classifier head (summary page, "Approach": pure low-precision
 * classifier, stochastic rounding, no momentum, gradient computation fused with the SGD update,
 * label dimension chunked; arXiv abstract: "gradient fusion and chunking").
 *
 *   W        [L, D] row-major weight codes (BF16, E4M3 or MXFP4 rows per `wdtype`), updated IN PLACE.
 *   X        [B, D] row-major BF16 codes (encoder features). Read only.
 *   row_ptr  [B+1] int32, ids [nnz] int32: the positive labels of each sample in CSR form; set
 *            semantics (duplicates collapse, any order, empty rows allowed). Ids outside [0, L)
 *            are skipped and raise bit ELMO_FLAG_LABEL_RANGE in the workspace flags word;
 *            row_ptr must be non-decreasing with row_ptr[0] = 0 and row_ptr[B] = nnz (violations
 *            raise ELMO_FLAG_ROW_PTR). `nnz` is the host-side count.
 *   lr       SGD learning rate (cast to FP32 by the caller's value).
 *   seed, step  key the counter-based RNG of the stochastic rounding: Philox4x32-10 with key =
 *            seed, counter = (g, step); element idx = j*D + k belongs to block g = idx >> 3 at
 *            position p = idx & 7, which takes 16-bit half p & 1 of output word p >> 1. Calling
 *            with the same (seed, step) on the same inputs reproduces the same W bit for bit,
 *            whatever the chunk size.
 *   chunk    labels per chunk: bounds the transient G buffer to B_pad * chunk * 2 bytes.
 *   dX       [B, D] FP32, OVERWRITTEN with sum_j G[b, j] * W_old[j, :] (pre-update weights).
 *   loss_sum nullable; if given, receives the FP32 value of the summed BCE over all (b, j).
 *   workspace, workspace_bytes: at least elmo_xmc_step_workspace_bytes(...) bytes of device
 *            memory, used for label buckets, padded/cast copies of X, one chunk of G and the dX
 *            partial sums. Its first 4 bytes are the flags word after the step completes.
 * Per element: z = X~ . w_j (X~ = X, or E4M3-RNE(X) for E4M3 and MXFP4 weights), g =
 * BF16-RNE(sigmoid(z) - y), dX += g W_old, dW = g^T X, t = fmaf(-lr, dW, w), W = SR(t) (for MXFP4
 * per 32-element block, as described with the formats).
 * Kernels: the faster of the two implementations for the shape: the single-pass step of
 * elmo_xmc_step_single_pass where it is built (B <= 32 and D = 256, 512 or 768), else the
 * two-kernel step of elmo_xmc_step_two_kernel. Both follow the rule above with the same random
 * bits; they sum each logit in a different order (see elmo_xmc_step_single_pass).
 */
#define ELMO_FLAG_LABEL_RANGE 1u
#define ELMO_FLAG_ROW_PTR 2u
size_t elmo_xmc_step_workspace_bytes(int B, int D, int64_t L, int64_t chunk, int wdtype,
                                     int64_t max_nnz);
int elmo_xmc_step(void* W, int wdtype, int64_t L, int D, const void* X, int B,
                  const int32_t* row_ptr, const int32_t* ids, int64_t nnz, float lr, uint64_t seed,
                  uint64_t step, int64_t chunk, float* dX, float* loss_sum, void* workspace,
                  size_t workspace_bytes, void* stream);
/*
 * The step as two kernels per label chunk, for every supported shape (summary page, "Approach":
 * the label dimension chunked, the gradient fused with the SGD update): a forward kernel writes the
 * chunk's BF16 gradient G (the one chunk-sized transient), then a backward kernel computes dX and
 * dW from it and updates the weights in place, dW never leaving its registers. Arguments,
 * workspace, results and errors as elmo_xmc_step, which takes this path for B > 32 or D not in
 * {256, 512, 768}.
 */
int elmo_xmc_step_two_kernel(void* W, int wdtype, int64_t L, int D, const void* X, int B,
                             const int32_t* row_ptr, const int32_t* ids, int64_t nnz, float lr,
                             uint64_t seed, uint64_t step, int64_t chunk, float* dX, float* loss_sum,
                             void* workspace, size_t workspace_bytes, void* stream);
/*
 * The same step as elmo_xmc_step computed in a single pass over the weights (summary page,
 * "Approach": the classifier gradient fused with the SGD update; arXiv abstract: "gradient
 * fusion"): one kernel per label chunk holds each 32-label weight tile in LDS while it computes the
 * tile's logits, its gradient G (kept on chip), the tile's share of dX and the update, so the
 * weights are read once and written once and no chunk of G goes to device memory. Built for
 * B <= 32 and D = 256, 512 or 768 (every weight format): there each work-group keeps its B x D FP32
 * dX accumulator in registers for the whole chunk; other shapes return ELMO_EUNSUPPORTED and
 * enqueue nothing. Arguments, workspace (elmo_xmc_step_workspace_bytes), results and errors as
 * elmo_xmc_step; the weights follow the same rule with the same random bits. Logits are summed in
 * a different order than in elmo_xmc_step, so a gradient code can round the other way and move its
 * row's updated weights; both paths meet the same tolerances against the rule.
 *   g_out    nullable diagnostic: if given, [B, L] uint16 (2-byte aligned), receives the BF16
 *            gradient codes the step used (costs a write of 2 B L bytes); otherwise untouched.
 */
int elmo_xmc_step_single_pass(void* W, int wdtype, int64_t L, int D, const void* X, int B,
                              const int32_t* row_ptr, const int32_t* ids, int64_t nnz, float lr,
                              uint64_t seed, uint64_t step, int64_t chunk, float* dX,
                              float* loss_sum, uint16_t* g_out, void* workspace,
                              size_t workspace_bytes, void* stream);
/*
 * The same step for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): arguments, results and errors as elmo_xmc_step,
 * with the workspace replaced by a static device array of ELMO_NOALLOC_SCRATCH_BYTES bytes inside
 * the library (one per GPU, held from the library's first use of that GPU until the process ends;
 * its address is looked up on the first call on each device). No device memory is allocated or
 * freed. A step whose workspace (elmo_xmc_step_workspace_bytes) exceeds that size returns
 * ELMO_ESCRATCH and enqueues nothing: at B = 256, D = 768 that allows chunks of up to about
 * 131,072 labels (3M-label E4M3 step: 97 MB); at B = 128, D = 768, chunks of 262,144 BF16 labels.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU (other streams or
 * threads) race and give undefined results; serialise them. The flags word is not readable here.
 * It runs the two-kernel step (elmo_xmc_step_two_kernel) for every shape.
 */
#define ELMO_NOALLOC_SCRATCH_BYTES (128u << 20)
int elmo_xmc_step_noalloc(void* W, int wdtype, int64_t L, int D, const void* X, int B,
                          const int32_t* row_ptr, const int32_t* ids, int64_t nnz, float lr,
                          uint64_t seed, uint64_t step, int64_t chunk, float* dX, float* loss_sum,
                          void* stream);

/* Copies the flags word of a step's workspace to *flags (HOST pointer); synchronises `stream`. */
int elmo_xmc_step_flags(const void* workspace, uint32_t* flags, void* stream);

/*
 * Top-k scoring for precision@k (summary page, "Experimental setup": P@1, P@3, P@5).
 *   W [L, D] codes, X [N, D] BF16 codes (E4M3 and MXFP4 weights score against E4M3-RNE(X), as in
 *   training).
 *   out_idx [N, k] int32: labels ranked by (FP32 logit desc, label asc), NaN logits last.
 *   out_score [N, k] FP32 logits, nullable.  1 <= k <= min(ELMO_MAX_TOPK, L), N >= 1.
 */
size_t elmo_xmc_topk_workspace_bytes(int N, int D, int64_t L, int k, int wdtype);
int elmo_xmc_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k,
                  int32_t* out_idx, float* out_score, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Diagnostic: FP32 logits Z [B, l1 - l0] (row-major) of labels [l0, l1) computed by the same
 * forward kernel the step uses. Workspace as for elmo_xmc_step with chunk = l1 - l0, nnz = 0.
 */
int elmo_xmc_logits(const void* W, int wdtype, int64_t L, int D, int64_t l0, int64_t l1,
                    const void* X, int B, float* Z, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Diagnostic: the step's forward kernel over labels [l0, l1) with the step's label handling,
 * writing the FP32 logits Z and/or the BF16 gradient codes G = BF16(sigmoid(Z) - Y) that a
 * two-kernel step with the same inputs uses (each [B, l1 - l0] row-major, nullable but not both;
 * the single-pass step reports its own codes through its g_out). Weights are not
 * touched. Labels as for elmo_xmc_step (row_ptr/ids may be NULL when nnz = 0). Workspace as for
 * elmo_xmc_step with chunk = l1 - l0 and max_nnz = nnz.
 */
int elmo_xmc_forward(const void* W, int wdtype, int64_t L, int D, const void* X, int B,
                     const int32_t* row_ptr, const int32_t* ids, int64_t nnz, int64_t l0, int64_t l1,
                     float* Z, uint16_t* G, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement aid (off by default; process-wide, not thread-safe): while enabled, each launch of
 * the step's forward (index 0) and backward/update (index 1) kernels is bracketed by HIP events on
 * the launch stream. elmo_xmc_kernel_timing_read waits for the recorded events and fills, for each
 * of the two kernels (HOST arrays of 2): summed milliseconds, number of launches and labels
 * processed; the records are then cleared.
 */
int elmo_xmc_kernel_timing(int enable);
int elmo_xmc_kernel_timing_read(double* ms, int64_t* launches, double* labels);

/* Kahan-compensated BF16 update of n encoder parameters, in place (ELMO summary, Approach: the
 * encoder is trained with Kahan summation and no FP32 master weights; the pages fix neither the
 * compensation's precision nor the order of operations, this is one step of Kahan's compensated
 * summation of the increments). w[i]: the parameter, c[i]: its compensation, both BF16 codes;
 * g[i]: the binary32 gradient. Per element, in binary32 with both stores rounded to nearest-even:
 *   d = -lr g;  y = d - c;  t = bf16(w + y);  c = bf16((t - w) - y);  w = t.
 * w, c, g: DEVICE pointers to n elements each, naturally aligned (2, 2, 4 bytes; 16-byte alignment
 * of all three takes the vector path), owned by the caller; w and c must not overlap each other or
 * g. n = 0 is a no-op. Returns ELMO_ESHAPE for n < 0, ELMO_EINVAL for a null or misaligned
 * pointer, ELMO_EHIP on a launch failure; asynchronous on `stream`. */
int elmo_kahan_update(uint16_t* w, uint16_t* c, const float* g, int64_t n, float lr, void* stream);

/*
 * Test hook: the device codec, stochastic rounding and RNG applied elementwise to n elements.
 *   op 0  BF16 RNE encode:      in0 float[n]            -> out uint16[n]
 *   op 1  E4M3 RNE-sat encode:  in0 float[n]            -> out uint8[n]
 *   op 2  E4M3 decode:          in0 uint8[n]            -> out float[n]
 *   op 3  SR to BF16:           in0 float[n], in1 uint32 r[n] -> out uint16[n]
 *   op 4  SR to E4M3:           in0 float[n], in1 uint32 r[n] -> out uint8[n]
 *   op 5  RNG 16-bit draws:     r16(seed, step, idx0 + i), idx0 = *(const uint64_t*)in0 (HOST) -> out uint32[n]
 *   op 6  gradient code:        in0 float z[n], in1 uint32 y[n] -> out uint16[n] (BF16(sigmoid(z) - y))
 *   op 7  E4M3 -> BF16, 4 codes per word as the backward kernel decodes its weight tiles:
 *                               in0 uint32[n] -> out uint32[2n] (BF16 pairs of bytes 0,1 and 2,3)
 *   op 8  gradient, the forward's small-argument form (meant for |z| <= 2), binary32 before rounding:
 *                               in0 float z[n], in1 uint32 y[n] -> out float[n]
 *   op 9  gradient, the forward's split-exponent form (meant for |z| <= 80), binary32 before rounding:
 *                               in0 float z[n], in1 uint32 y[n] -> out float[n]
 *   op 10 SR to E2M1 (v already divided by its block scale): in0 float[n], in1 uint32 r[n] -> out uint8[n]
 *   op 11 MX block quantisation: in0 float t[32 n], in1 uint32 r[32 n] -> out uint8[33 n] (per block the
 *                               32 E2M1 codes, then the E8M0 scale code; 255 for a block with a NaN)
 *   op 12 E2M1 -> BF16 as the backward decodes MXFP4 weight tiles: in0 uint32 w[n] (8 codes, low
 *                               nibble first), in1 uint32 E8M0 scale code[n] -> out uint32[4 n] (BF16 pairs)
 *   op 13 one scaled MFMA in the forward's MXFP4 operand layout (E4M3 A, E2M1 B, E8M0 scales per
 *                               32-element block): in0 uint8[3200] = A codes [32][64], B codes [32][32]
 *                               (two per byte), A scales [32][2], B scales [32][2]; out float[1024] = C
 *                               [32][32] row-major; n must be 1
 *   op 14 the device's scaled FP4 conversion with stochastic rounding (a test hook for its rounding
 *                               rule): in0 float[2n] pairs, in1 uint32[2n] (random operand, scale
 *                               bits) per pair -> out uint32[n] (the two codes in byte 0)
 */
int elmo_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n,
                        uint64_t seed, uint64_t step, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ELMO_XMC_H */
