// Elementwise application of the device codec, stochastic rounding, RNG and gradient rule, so that
// tests can compare them bit for bit with an independent implementation.
#include "mfma.hpp"
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
      case 10: {
        ((uint8_t*)out)[i] = (uint8_t)sr_e2m1_scaled(((const float*)in0)[i], 1.0f, ((const uint32_t*)in1)[i] << 16);
        break;
      }
      case 11: {
        // one MX block per element i: 32 FP32 values and draws -> 32 codes and the scale code
        const float* t = (const float*)in0 + 32 * i;
        const uint32_t* r = (const uint32_t*)in1 + 32 * i;
        uint8_t* o = (uint8_t*)out + 33 * i;
        float amax = 0.0f;
        bool nan = false;
        for (int k = 0; k < 32; ++k) { nan |= t[k] != t[k]; amax = fmaxf(amax, __builtin_fabsf(t[k])); }
        if (nan) {
          for (int k = 0; k < 32; ++k) o[k] = 0;
          o[32] = 255;
        } else {
          const int x = mx_block_exponent(amax);
          const float sc = e8m0_to_f32((uint32_t)(x + 127));
          for (int k = 0; k < 32; ++k) o[k] = (uint8_t)sr_e2m1_scaled(t[k], sc, r[k] << 16);
          o[32] = (uint8_t)(x + 127);
        }
        break;
      }
      case 14: {
        // the scaled FP4 conversion with stochastic rounding as it stands: the float pair in0[2i],
        // in0[2i+1], random operand in1[2i], scale bits in1[2i+1] -> the result word
        const f32x2_t v = {((const float*)in0)[2 * i], ((const float*)in0)[2 * i + 1]};
        const uint32_t* r = (const uint32_t*)in1 + 2 * i;
        ((uint32_t*)out)[i] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v, r[0], u2f(r[1]), 0);
        break;
      }
      case 12: {
        // 8 E2M1 codes (4 bytes) with E8M0 scale in1[i] -> 4 BF16 pairs (bytes 0 .. 3)
        const uint32_t w = ((const uint32_t*)in0)[i];
        const float sc = e8m0_to_f32(((const uint32_t*)in1)[i]);
        uint32_t* o = (uint32_t*)out + 4 * i;
        o[0] = fp4x2_to_bf16x2<0>(w, sc); o[1] = fp4x2_to_bf16x2<1>(w, sc);
        o[2] = fp4x2_to_bf16x2<2>(w, sc); o[3] = fp4x2_to_bf16x2<3>(w, sc);
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

// One 32 x 32 x 64 scaled MFMA with E4M3 A and E2M1 B operands and per-lane E8M0 block scales, in
// the operand layouts the forward uses: lane l holds A row l % 32 and B column l % 32, K values
// 32 (l / 32) .. + 31 (32 bytes of A, 16 bytes of B with element 2e in the low nibble of byte e), and
// the scales of those 32-element K blocks. in: A codes [32][64], B codes [32][32] (two per byte),
// scale codes A [32][2], B [32][2]; out: C [32][32] FP32 row-major.
__global__ void k_mx_mfma_probe(const uint8_t* __restrict__ in, float* __restrict__ out) {
  const int lane = threadIdx.x, l32 = lane & 31, hi = lane >> 5;
  const uint8_t* A = in;
  const uint8_t* Bm = in + 2048;
  const uint8_t* sA = in + 3072;
  const uint8_t* sB = in + 3136;
  // the E4M3 operand beside an FP4 one: bytes 0-15 hold k = 16 hi + e, bytes 16-31 k = 32 + 16 hi + e
  const i32x4_t a0 = *(const i32x4_t*)(A + l32 * 64 + hi * 16), a1 = *(const i32x4_t*)(A + l32 * 64 + 32 + hi * 16);
  const i32x4_t b0 = *(const i32x4_t*)(Bm + l32 * 32 + hi * 16);
  const i32x8_t av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const i32x8_t bv = {b0[0], b0[1], b0[2], b0[3], 0, 0, 0, 0};
  const f32x16_t c = mfma_e4m3_fp4(av, bv, f32x16_t{}, (int)sA[l32 * 2 + hi], (int)sB[l32 * 2 + hi]);
#pragma unroll
  for (int i = 0; i < 16; ++i) out[(8 * (i >> 2) + 4 * hi + (i & 3)) * 32 + l32] = c[i];
}

int run_numerics_probe(int op, const void* in0, const void* in1, void* out, int64_t n, uint64_t seed,
                       uint64_t step, hipStream_t st) {
  if (op < 0 || op > 14 || n < 0 || !out) return ELMO_EINVAL_;
  if (op != 5 && !in0) return ELMO_EINVAL_;
  if ((op == 3 || op == 4 || op == 6 || op == 8 || op == 9 || op == 10 || op == 11 || op == 12 || op == 14) && !in1)
    return ELMO_EINVAL_;
  if (n == 0) return ELMO_OK_;
  if (op == 13) {
    hipLaunchKernelGGL(k_mx_mfma_probe, dim3(1), dim3(64), 0, st, (const uint8_t*)in0, (float*)out);
    return hipGetLastError() == hipSuccess ? ELMO_OK_ : ELMO_EHIP_;
  }
  uint64_t idx0 = 0;
  if (op == 5) idx0 = in0 ? *(const uint64_t*)in0 : 0;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_numerics, dim3((unsigned)blocks), dim3(256), 0, st, op, op == 5 ? nullptr : in0, in1, out, n,
                     seed, step, idx0);
  return hipGetLastError() == hipSuccess ? ELMO_OK_ : ELMO_EHIP_;
}

}  // namespace elmo
