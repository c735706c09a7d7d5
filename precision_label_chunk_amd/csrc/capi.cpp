// C ABI of the elmo_xmc library (declared in include/elmo_xmc.h): argument validation on the host,
// then the internal launchers. Nothing here allocates device memory or synchronises, except
// elmo_xmc_step_flags, which copies one word back by design.
#include "../../include/elmo_xmc.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "step_kernels.hpp"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// the weight format, and the feature sizes it supports (MXFP4 rows must be 8-byte aligned)
int check_format(int wdtype, int D) {
  if (wdtype != ELMO_W_BF16 && wdtype != ELMO_W_E4M3 && wdtype != ELMO_W_MXFP4) return ELMO_EDTYPE;
  if (wdtype == ELMO_W_MXFP4 && D % 256 != 0) return ELMO_ESHAPE;
  return ELMO_OK;
}

int check_shapes(int B, int D, int64_t L) {
  if (B < 1 || B > ELMO_MAX_B) return ELMO_ESHAPE;
  if (D < 64 || D > ELMO_MAX_D || D % 64 != 0) return ELMO_ESHAPE;
  if (L < 1 || L >= (int64_t(1) << 31)) return ELMO_ESHAPE;
  return ELMO_OK;
}

// which kernels a step runs: the faster for its shape (the single pass where it is built, B <= 32
// and D = 256, 512 or 768), or the one the caller names
enum { PATH_AUTO = 0, PATH_TWO_KERNEL = 1, PATH_SINGLE = 2 };

int step_entry(void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
               const int32_t* ids, int64_t nnz, float lr, uint64_t seed, uint64_t step, int64_t chunk, float* dX,
               float* loss_sum, uint16_t* g_out, void* workspace, size_t workspace_bytes, void* stream,
               int path) {
  int rc = check_format(wdtype, D);
  if (rc != ELMO_OK) return rc;
  if ((rc = check_shapes(B, D, L)) != ELMO_OK) return rc;
  if (chunk < 1 || nnz < 0 || !std::isfinite(lr)) return ELMO_EINVAL;
  if (!W || !X || !row_ptr || !dX || (nnz > 0 && !ids)) return ELMO_EINVAL;
  if (!aligned16(W) || !aligned16(X) || !aligned16(dX)) return ELMO_EINVAL;
  const bool fits = elmo::single_pass_shape(elmo::padded_batch(B), D);
  if (path == PATH_SINGLE && !fits) return ELMO_EUNSUPPORTED;
  const bool single = path == PATH_SINGLE || (path == PATH_AUTO && fits);
  if (!workspace || !aligned16(workspace)) return ELMO_EWORKSPACE;
  const elmo::StepLayout s = elmo::step_layout(B, D, L, chunk, wdtype, nnz);
  if (workspace_bytes < s.total) return ELMO_EWORKSPACE;
  elmo::StepArgs a{};
  a.W = W; a.wdtype = wdtype; a.L = L; a.D = D; a.X = X; a.B = B;
  a.row_ptr = row_ptr; a.ids = ids; a.nnz = nnz; a.lr = lr; a.seed = seed; a.step = step;
  a.dX = dX; a.loss = loss_sum; a.l0 = 0; a.l1 = L; a.Z = nullptr; a.single = single;
  a.Gout = g_out;                        // (single pass only: its diagnostic gradient copy)
  return elmo::run_step(a, s, workspace, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int elmo_abi_version(void) { return 1; }

const char* elmo_status_str(int status) {
  switch (status) {
    case ELMO_OK: return "ok";
    case ELMO_EINVAL: return "invalid argument";
    case ELMO_ESHAPE: return "unsupported shape";
    case ELMO_EDTYPE: return "unknown weight format";
    case ELMO_EWORKSPACE: return "workspace missing or too small";
    case ELMO_EHIP: return "HIP runtime error";
    case ELMO_EUNSUPPORTED: return "not supported by this library";
    case ELMO_ESCRATCH: return "step needs more scratch than the allocation-free entry point's static buffer holds";
    default: return "unknown status";
  }
}

size_t elmo_xmc_step_workspace_bytes(int B, int D, int64_t L, int64_t chunk, int wdtype, int64_t max_nnz) {
  if (check_shapes(B, D, L) != ELMO_OK || chunk < 1 || max_nnz < 0) return 0;
  if (check_format(wdtype, D) != ELMO_OK) return 0;
  return elmo::step_layout(B, D, L, chunk, wdtype, max_nnz).total;
}

int elmo_xmc_step(void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
                  const int32_t* ids, int64_t nnz, float lr, uint64_t seed, uint64_t step, int64_t chunk,
                  float* dX, float* loss_sum, void* workspace, size_t workspace_bytes, void* stream) {
  return step_entry(W, wdtype, L, D, X, B, row_ptr, ids, nnz, lr, seed, step, chunk, dX, loss_sum, nullptr,
                    workspace, workspace_bytes, stream, PATH_AUTO);
}

int elmo_xmc_step_two_kernel(void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
                             const int32_t* ids, int64_t nnz, float lr, uint64_t seed, uint64_t step, int64_t chunk,
                             float* dX, float* loss_sum, void* workspace, size_t workspace_bytes, void* stream) {
  return step_entry(W, wdtype, L, D, X, B, row_ptr, ids, nnz, lr, seed, step, chunk, dX, loss_sum, nullptr,
                    workspace, workspace_bytes, stream, PATH_TWO_KERNEL);
}

int elmo_xmc_step_single_pass(void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
                              const int32_t* ids, int64_t nnz, float lr, uint64_t seed, uint64_t step,
                              int64_t chunk, float* dX, float* loss_sum, uint16_t* g_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (g_out && ((uintptr_t)g_out & 1u)) return ELMO_EINVAL;
  return step_entry(W, wdtype, L, D, X, B, row_ptr, ids, nnz, lr, seed, step, chunk, dX, loss_sum, g_out,
                    workspace, workspace_bytes, stream, PATH_SINGLE);
}

int elmo_xmc_step_noalloc(void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
                          const int32_t* ids, int64_t nnz, float lr, uint64_t seed, uint64_t step, int64_t chunk,
                          float* dX, float* loss_sum, void* stream) {
  int rc = check_format(wdtype, D);
  if (rc != ELMO_OK) return rc;
  if ((rc = check_shapes(B, D, L)) != ELMO_OK) return rc;
  if (chunk < 1 || nnz < 0 || !std::isfinite(lr)) return ELMO_EINVAL;
  if (!W || !X || !row_ptr || !dX || (nnz > 0 && !ids)) return ELMO_EINVAL;
  if (!aligned16(W) || !aligned16(X) || !aligned16(dX)) return ELMO_EINVAL;
  const elmo::StepLayout s = elmo::step_layout(B, D, L, chunk, wdtype, nnz);
  if (s.total > (size_t)ELMO_NOALLOC_SCRATCH_BYTES) return ELMO_ESCRATCH;
  void* ws = nullptr;
  if ((rc = elmo::noalloc_scratch(&ws)) != ELMO_OK) return rc;
  elmo::StepArgs a{};
  a.W = W; a.wdtype = wdtype; a.L = L; a.D = D; a.X = X; a.B = B;
  a.row_ptr = row_ptr; a.ids = ids; a.nnz = nnz; a.lr = lr; a.seed = seed; a.step = step;
  a.dX = dX; a.loss = loss_sum; a.l0 = 0; a.l1 = L; a.Z = nullptr;
  return elmo::run_step(a, s, ws, (hipStream_t)stream);
}

int elmo_xmc_step_flags(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return ELMO_EINVAL;
  if (hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
    return ELMO_EHIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return ELMO_EHIP;
  return ELMO_OK;
}

int elmo_xmc_forward(const void* W, int wdtype, int64_t L, int D, const void* X, int B, const int32_t* row_ptr,
                     const int32_t* ids, int64_t nnz, int64_t l0, int64_t l1, float* Z, uint16_t* G,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_format(wdtype, D);
  if (rc != ELMO_OK) return rc;
  if ((rc = check_shapes(B, D, L)) != ELMO_OK) return rc;
  if (l0 < 0 || l1 > L || l1 <= l0) return ELMO_ESHAPE;
  if (nnz < 0 || (nnz > 0 && (!ids || !row_ptr))) return ELMO_EINVAL;
  if (!W || !X || (!Z && !G) || !aligned16(W) || !aligned16(X)) return ELMO_EINVAL;
  if (!workspace || !aligned16(workspace)) return ELMO_EWORKSPACE;
  const elmo::StepLayout s = elmo::step_layout(B, D, L, l1 - l0, wdtype, nnz);
  if (workspace_bytes < s.total) return ELMO_EWORKSPACE;
  elmo::StepArgs a{};
  a.W = const_cast<void*>(W); a.wdtype = wdtype; a.L = L; a.D = D; a.X = X; a.B = B;
  a.row_ptr = row_ptr; a.ids = ids; a.nnz = nnz;
  a.l0 = l0 - l0 % elmo::TJ1; a.l1 = l1;
  a.Z = Z; a.Gout = G; a.zpitch = l1 - l0; a.zoff = l0;
  return elmo::run_step(a, s, workspace, (hipStream_t)stream);
}

int elmo_xmc_logits(const void* W, int wdtype, int64_t L, int D, int64_t l0, int64_t l1, const void* X, int B,
                    float* Z, void* workspace, size_t workspace_bytes, void* stream) {
  if (!Z) return ELMO_EINVAL;
  return elmo_xmc_forward(W, wdtype, L, D, X, B, nullptr, nullptr, 0, l0, l1, Z, nullptr, workspace,
                          workspace_bytes, stream);
}

size_t elmo_xmc_topk_workspace_bytes(int N, int D, int64_t L, int k, int wdtype) {
  if (N < 1 || D < 64 || D > ELMO_MAX_D || D % 64 != 0 || L < 1 || L >= (int64_t(1) << 31)) return 0;
  if (k < 1 || k > ELMO_MAX_TOPK || k > L) return 0;
  if (check_format(wdtype, D) != ELMO_OK) return 0;
  return elmo::topk_layout(N, D, L, k, wdtype).total;
}

int elmo_xmc_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k, int32_t* out_idx,
                  float* out_score, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_format(wdtype, D);
  if (rc != ELMO_OK) return rc;
  if (N < 1 || D < 64 || D > ELMO_MAX_D || D % 64 != 0 || L < 1 || L >= (int64_t(1) << 31)) return ELMO_ESHAPE;
  if (k < 1 || k > ELMO_MAX_TOPK || k > L) return ELMO_ESHAPE;
  if (!W || !X || !out_idx || !aligned16(W) || !aligned16(X)) return ELMO_EINVAL;
  if (!workspace || !aligned16(workspace)) return ELMO_EWORKSPACE;
  const elmo::TopkLayout s = elmo::topk_layout(N, D, L, k, wdtype);
  if (workspace_bytes < s.total) return ELMO_EWORKSPACE;
  return elmo::run_topk(W, wdtype, L, D, X, N, k, out_idx, out_score, s, workspace, (hipStream_t)stream);
}

int elmo_xmc_kernel_timing(int enable) {
  elmo::kernel_timing_enable(enable);
  return ELMO_OK;
}

int elmo_xmc_kernel_timing_read(double* ms, int64_t* launches, double* labels) {
  if (!ms || !launches || !labels) return ELMO_EINVAL;
  return elmo::kernel_timing_read(ms, launches, labels);
}

int elmo_kahan_update(uint16_t* w, uint16_t* c, const float* g, int64_t n, float lr, void* stream) {
  if (n < 0) return ELMO_ESHAPE;
  if (n == 0) return ELMO_OK;
  if (!w || !c || !g || (uintptr_t)w % 2 || (uintptr_t)c % 2 || (uintptr_t)g % 4) return ELMO_EINVAL;
  return elmo::run_kahan_update(w, c, g, n, lr, (hipStream_t)stream);
}

int elmo_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n, uint64_t seed,
                        uint64_t step, void* stream) {
  return elmo::run_numerics_probe(op, in0, in1, out, n, seed, step, (hipStream_t)stream);
}

}  // extern "C"
