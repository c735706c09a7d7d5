// Kahan-compensated BF16 update of the encoder's parameters (ELMO summary, Approach: the encoder is
// trained with Kahan summation and no FP32 master weights). Each parameter w is a BF16 code with a
// BF16 compensation c beside it; one update is one step of Kahan's compensated summation of the
// increments d = -lr g, evaluated in binary32 with the two stores rounded to nearest-even:
//   y = d - c,  t = bf16(w + y),  c = bf16((t - w) - y),  w = t.
// The work is elementwise and bound by HBM (12 bytes per parameter: w, c and g read, w and c
// written): 8 parameters per thread with 16-byte non-temporal accesses when the three arrays allow
// it, up to 256 work-groups per CU (one pass for an encoder-sized array), a scalar tail.
#include "mfma.hpp"
#include "numerics.hpp"
#include "step_kernels.hpp"

namespace elmo {

__device__ __forceinline__ void kahan1(uint32_t wb, uint32_t cb, float g, float lr, uint32_t& wo, uint32_t& co) {
  const float w = bf16_to_f32(wb), c = bf16_to_f32(cb);
  const float d = -lr * g;
  const float y = d - c;
  const uint32_t t = f32_to_bf16_rne(w + y);
  co = f32_to_bf16_rne((bf16_to_f32(t) - w) - y);
  wo = t;
}

// vector form: parameters 8 i .. 8 i + 7 for i < n8; the last n % 8 by the scalar form
__global__ __launch_bounds__(256) void k_kahan8(uint16_t* __restrict__ w, uint16_t* __restrict__ c,
                                                const float* __restrict__ g, int64_t n8, float lr) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    // (every byte is touched once: non-temporal accesses keep the stream from displacing the caches)
    const i32x4_t wv = __builtin_nontemporal_load((const i32x4_t*)w + i);
    const i32x4_t cv = __builtin_nontemporal_load((const i32x4_t*)c + i);
    const f32x4_t g0 = __builtin_nontemporal_load((const f32x4_t*)g + 2 * i);
    const f32x4_t g1 = __builtin_nontemporal_load((const f32x4_t*)g + 2 * i + 1);
    const uint32_t wa[4] = {(uint32_t)wv[0], (uint32_t)wv[1], (uint32_t)wv[2], (uint32_t)wv[3]};
    const uint32_t ca[4] = {(uint32_t)cv[0], (uint32_t)cv[1], (uint32_t)cv[2], (uint32_t)cv[3]};
    const float ga[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    uint32_t wo[4], co[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t w0, c0, w1, c1;
      kahan1(wa[k] & 0xffffu, ca[k] & 0xffffu, ga[2 * k], lr, w0, c0);
      kahan1(wa[k] >> 16, ca[k] >> 16, ga[2 * k + 1], lr, w1, c1);
      wo[k] = w0 | (w1 << 16);
      co[k] = c0 | (c1 << 16);
    }
    __builtin_nontemporal_store(i32x4_t{(int)wo[0], (int)wo[1], (int)wo[2], (int)wo[3]}, (i32x4_t*)w + i);
    __builtin_nontemporal_store(i32x4_t{(int)co[0], (int)co[1], (int)co[2], (int)co[3]}, (i32x4_t*)c + i);
  }
}

__global__ __launch_bounds__(256) void k_kahan1(uint16_t* __restrict__ w, uint16_t* __restrict__ c,
                                                const float* __restrict__ g, int64_t i0, int64_t n, float lr) {
  for (int64_t i = i0 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t wo, co;
    kahan1(w[i], c[i], g[i], lr, wo, co);
    w[i] = (uint16_t)wo;
    c[i] = (uint16_t)co;
  }
}

int run_kahan_update(uint16_t* w, uint16_t* c, const float* g, int64_t n, float lr, hipStream_t st) {
  if (n == 0) return ELMO_OK_;
  const bool vec = ((uintptr_t)w % 16 == 0) && ((uintptr_t)c % 16 == 0) && ((uintptr_t)g % 16 == 0);
  const int64_t n8 = vec ? n / 8 : 0;
  const int cap = 256 * device_cus();          // (many short-lived work-groups stream best)
  if (n8 > 0) {
    const int64_t want = (n8 + 255) / 256;
    hipLaunchKernelGGL(k_kahan8, dim3((unsigned)(want < cap ? want : cap)), dim3(256), 0, st, w, c, g, n8, lr);
    if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  }
  if (8 * n8 < n) {
    const int64_t want = (n - 8 * n8 + 255) / 256;
    hipLaunchKernelGGL(k_kahan1, dim3((unsigned)(want < cap ? want : cap)), dim3(256), 0, st, w, c, g, 8 * n8, n, lr);
    if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  }
  return ELMO_OK_;
}

}  // namespace elmo
