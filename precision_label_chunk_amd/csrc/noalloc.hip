// Static scratch memory for the training step's allocation-free entry point
// (elmo_xmc_step_noalloc in capi.cpp), for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation.
//
// The step's scratch (label buckets, the padded and cast copies of X, one chunk of gradient codes,
// the dX partial sums, the flags word) lives in one file-scope device array of
// ELMO_NOALLOC_SCRATCH_BYTES bytes, which every GPU that loads the library holds until the process
// ends. Its device address is looked up once per device (hipGetSymbolAddress, with that device
// current) on the first call there and kept; host code passes that address to the kernels, never
// the array's name. The array keeps the last call's contents, and calls that overlap on one GPU
// share it, so they race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/elmo_xmc.h"
#include "step_kernels.hpp"

namespace elmo {

static __device__ __align__(256) uint8_t scratch[ELMO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

}  // namespace

int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ELMO_EHIP_;
  if (dev < 0 || dev >= MAX_DEVICES) return ELMO_EUNSUPPORTED_;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ELMO_EHIP_;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return ELMO_OK_;
}

}  // namespace elmo
