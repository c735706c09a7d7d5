// Elementwise application of the device codec, stochastic rounding, RNG and gradient rule, so that
// tests can compare them bit for bit with an independent implementation.
#include "numerics.hpp"
#include "step_kernels.hpp"

namespace elmo {

__global__ void k_numerics(int op, const void* __restrict__ in0, const void* __restrict__ in1,
                           void* __restrict__ out, int64_t n, uint64_t seed, uint64_t step, uint64_t idx0) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    switch (op) {
      case 0: ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_rne(((const float*)in0)[i]); break;
      case 1: ((uint8_t*)out)[i] = (uint8_t)f32_to_e4m3_rne_sat(((const float*)in0)[i]); break;
      case 2: ((float*)out)[i] = e4m3_to_f32(((const uint8_t*)in0)[i]); break;
      case 3: ((uint16_t*)out)[i] = (uint16_t)sr_bf16(((const float*)in0)[i], ((const uint32_t*)in1)[i] & 0xffffu); break;
      case 4: ((uint8_t*)out)[i] = (uint8_t)sr_e4m3(((const float*)in0)[i], ((const uint32_t*)in1)[i] & 0xffffu); break;
      case 5: {
        const uint64_t idx = idx0 + (uint64_t)i;
        ((uint32_t*)out)[i] = rng_r16(seed, step, idx);
        break;
      }
      case 6: {
        const float z = ((const float*)in0)[i];
        const bool y = ((const uint32_t*)in1)[i] != 0;
        ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_rne(bce_grad(z, y));
        break;
      }
      case 7: {
        uint32_t lo, hi;
        e4m3x4_to_bf16x4(((const uint32_t*)in0)[i], lo, hi);
        ((uint32_t*)out)[2 * i] = lo;
        ((uint32_t*)out)[2 * i + 1] = hi;
        break;
      }
      case 8:
      case 9: {
        const float z = ((const float*)in0)[i];
        const uint32_t ys = ((const uint32_t*)in1)[i] != 0 ? 0x80000000u : 0u;
        ((float*)out)[i] = op == 8 ? bce_grad_small_m(z, ys) : bce_grad_fast_m(z, ys);
        break;
      }
      default: break;
    }
  }
}

int run_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n, uint64_t seed,
                       uint64_t step, hipStream_t st) {
  if (op < 0 || op > 9 || n < 0 || !out) return ELMO_EINVAL_;
  if (op != 5 && !in0) return ELMO_EINVAL_;
  if ((op == 3 || op == 4 || op == 6 || op == 8 || op == 9) && !in1) return ELMO_EINVAL_;
  if (n == 0) return ELMO_OK_;
  uint64_t idx0 = 0;
  if (op == 5) idx0 = in0 ? *(const uint64_t*)in0 : 0;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_numerics, dim3((unsigned)blocks), dim3(256), 0, st, op, op == 5 ? nullptr : in0, in1, out, n,
                     seed, step, idx0);
  return hipGetLastError() == hipSuccess ? ELMO_OK_ : ELMO_EHIP_;
}

}  // namespace elmo
