// Internal interface between the C ABI (capi.cpp) and the HIP kernels of the XMC head step.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace elmo {

// status and format codes (mirror include/elmo_xmc.h)
constexpr int ELMO_OK_ = 0, ELMO_EINVAL_ = -1, ELMO_ESHAPE_ = -2, ELMO_EDTYPE_ = -3, ELMO_EWORKSPACE_ = -4,
              ELMO_EHIP_ = -5, ELMO_EUNSUPPORTED_ = -6;
constexpr int W_BF16_ = 0, W_E4M3_ = 1;
constexpr uint32_t ELMO_FLAG_LABEL_RANGE_ = 1u, ELMO_FLAG_ROW_PTR_ = 2u;

constexpr int TJ1 = 128;       // labels per forward tile (and label-bucket granularity)
constexpr int TJ2 = 64;        // labels per backward tile

struct StepLayout {
  int MB, DS, NS, NR;
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
  float* Z; uint16_t* Gout; int64_t zpitch; int64_t zoff;
  bool forward_only() const { return Z != nullptr || Gout != nullptr; }
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

// top-k
struct TopkLayout { int MB, NRg; int64_t ncand; size_t xb, xq, cand_s, cand_i, total; };
TopkLayout topk_layout(int N, int D, int64_t L, int k, int wdtype);
int run_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k, int32_t* idx,
             float* score, const TopkLayout& s, void* workspace, hipStream_t st);

// Kahan-compensated BF16 update of encoder parameters (elementwise)
int run_kahan_update(uint16_t* w, uint16_t* c, const float* g, int64_t n, float lr, hipStream_t st);

// elementwise numerics hook
int run_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n, uint64_t seed,
                       uint64_t step, hipStream_t st);

}  // namespace elmo
