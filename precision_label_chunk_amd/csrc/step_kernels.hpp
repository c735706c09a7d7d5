// Internal interface between the C ABI (capi.cpp) and the HIP kernels of the XMC head step.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace elmo {

// status and format codes (mirror include/elmo_xmc.h)
constexpr int ELMO_OK_ = 0, ELMO_EINVAL_ = -1, ELMO_ESHAPE_ = -2, ELMO_EDTYPE_ = -3, ELMO_EWORKSPACE_ = -4,
              ELMO_EHIP_ = -5, ELMO_EUNSUPPORTED_ = -6, ELMO_ESCRATCH_ = -7;
constexpr int W_BF16_ = 0, W_E4M3_ = 1, W_MXFP4_ = 2;
// bytes of one weight row: D codes (BF16, E4M3), or D/2 bytes of E2M1 code pairs then D/32 E8M0
// block scales (MXFP4)
__host__ __device__ constexpr int64_t w_row_bytes(int wf, int D) {
  return wf == W_BF16_ ? 2 * (int64_t)D : wf == W_E4M3_ ? (int64_t)D : (int64_t)D / 2 + D / 32;
}
constexpr uint32_t ELMO_FLAG_LABEL_RANGE_ = 1u, ELMO_FLAG_ROW_PTR_ = 2u;

constexpr int TJ1 = 128;       // labels per forward tile (and label-bucket granularity)
constexpr int TJ2 = 64;        // labels per backward tile

// The forward a step shape takes, and so the order the prepared feature copies are written in:
// features stationary in registers for E4M3 / MXFP4 weights at 256 padded samples and for BF16
// weights at 128, both at D = 768 (each lane's fragments then lie 1 KiB-contiguous per wave, in
// the order the kernel loads them), else the tiled forward over row-major copies.
constexpr int XLAY_ROWS = 0, XLAY_XS_E4M3 = 1, XLAY_XS_MX = 2, XLAY_XB = 3;
__host__ __device__ constexpr int fwd_x_layout(int MB, int wf, int D) {
  return D != 768 ? XLAY_ROWS
         : (MB == 256 && wf == W_E4M3_) ? XLAY_XS_E4M3
         : (MB == 256 && wf == W_MXFP4_) ? XLAY_XS_MX
         : (MB == 128 && wf == W_BF16_) ? XLAY_XB
                                        : XLAY_ROWS;
}

struct StepLayout {
  int MB, DS, NS, NR;
  int NR1;                              // single-pass work-groups (label ranges); 0 where not built
  int cus;                              // compute units of the device
  int64_t Cc, ntiles;
  size_t flags, tile_cnt, tile_off, bucket, xb, xq, xbt, g, part, loss, total;
};

struct StepArgs {
  void* W; int wdtype; int64_t L; int D; const void* X; int B;
  const int32_t* row_ptr; const int32_t* ids; int64_t nnz;
  float lr; uint64_t seed; uint64_t step;
  float* dX; float* loss;
  int64_t l0, l1;                       // label range processed (whole [0, L) for a step)
  // forward-only diagnostic: logits Z and/or gradient codes Gout, [B][zpitch] with column = label - zoff
  // (for the single-pass step, Gout is its optional copy of the gradient codes, [B][L])
  float* Z; uint16_t* Gout; int64_t zpitch; int64_t zoff;
  bool single;                          // the single-pass kernel instead of the two chunk kernels
  bool forward_only() const { return !single && (Z != nullptr || Gout != nullptr); }
};

// Optional per-launch HIP-event timing of the two chunk kernels (a measurement aid; off by default).
// When enabled, every forward / backward launch of a step is bracketed by events on the launch
// stream; kernel_timing_read() synchronises those events and returns the summed milliseconds.
enum { KT_FWD = 0, KT_BWD = 1 };
void kernel_timing_enable(int on);
int kernel_timing_read(double* ms, int64_t* launches, double* labels);
void kt_begin(int kind, hipStream_t st, int64_t labels);
void kt_end(int kind, hipStream_t st);

int padded_batch(int B);
int device_cus();
StepLayout step_layout(int B, int D, int64_t L, int64_t chunk, int wdtype, int64_t max_nnz);
int run_step(const StepArgs& a, const StepLayout& s, void* workspace, hipStream_t st);
// the per-chunk kernels of a step over labels [a.l0, a.l1) (step_chunks.hip, one object per <MB, WF>)
template <int MB, int WF>
int run_chunks(const StepArgs& a, const StepLayout& s, uint8_t* ws, hipStream_t st);
extern template int run_chunks<32, W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<64, W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<128, W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<256, W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<32, W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<64, W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<128, W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<256, W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<32, W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<64, W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<128, W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_chunks<256, W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);

// the single-pass step (step_single.hip): built for padded batches of 32 samples and D = 256, 512
// or 768
__host__ __device__ constexpr bool single_pass_shape(int MB, int D) { return MB == 32 && (D == 256 || D == 512 || D == 768); }
template <int WF>
int run_single(const StepArgs& a, const StepLayout& s, uint8_t* ws, hipStream_t st);
extern template int run_single<W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_single<W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
extern template int run_single<W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);

// top-k
struct TopkLayout { int MB, NRg; int64_t ncand; size_t xb, xq, cand_s, cand_i, total; };
TopkLayout topk_layout(int N, int D, int64_t L, int k, int wdtype);
int run_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k, int32_t* idx,
             float* score, const TopkLayout& s, void* workspace, hipStream_t st);

// Kahan-compensated BF16 update of encoder parameters (elementwise)
int run_kahan_update(uint16_t* w, uint16_t* c, const float* g, int64_t n, float lr, hipStream_t st);

// this device's copy of the static scratch array of the allocation-free step (noalloc.hip): its
// device address, looked up on the first call on the current device
int noalloc_scratch(void** out);

// elementwise numerics hook
int run_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n, uint64_t seed,
                       uint64_t step, hipStream_t st);

}  // namespace elmo
