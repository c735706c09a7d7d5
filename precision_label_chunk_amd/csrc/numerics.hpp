// Device numerics for the XMC head step on gfx950: BF16, OCP-E4M3 and MX-scaled FP4 (E2M1 with
// E8M0 block scales) codecs, stochastic rounding, the counter-based RNG that drives it, and the
// sigmoid-BCE gradient.
//
// Method context: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large Output
// Spaces" (summary page, "Approach" and "Surprising findings"): pure BF16/FP8-E4M3 classifier
// weights without master weights or tensor scaling, updated with stochastic rounding. The pages do
// not give the rounding mechanism or RNG; the rules implemented here are:
//   * RNE for X -> E4M3 and for G -> BF16; E4M3 encode saturates to +-448 (no infinity in E4M3FN);
//   * SR of an FP32 value t with 16 random bits r: keep the truncated magnitude, add one unit in
//     the last place iff (dropped fraction, as a 16-bit fixed-point number q) + r >= 2^16;
//   * r comes from Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3",
//     SC'11) with key = seed and counter = (g, step): the element indices 8g .. 8g + 7 share block
//     g = idx >> 3, and element idx = j*D + k takes 16-bit half (idx & 1) of output word
//     (idx >> 1) & 3 of its block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace elmo {

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---- BF16 -------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return u2f(h << 16); }

// round-to-nearest-even (v_cvt_pk_bf16_f32); NaN stays NaN
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// two values packed low / high, each rounded as above (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// ---- OCP E4M3 (E4M3FN) --------------------------------------------------------------------------
// gfx950's FP8 conversions use the OCP encoding (0x7E = 448, 0x7F/0xFF NaN, subnormals kept).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// the four E4M3 codes in the bytes of v as BF16 codes: lo = bytes 0 | 1 << 16, hi = bytes 2 | 3 << 16
// (gfx950's paired FP8 -> BF16 conversion with unit scale; exact: E4M3 values have at most 4
// significant bits and exponents inside BF16's range)
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t v, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v, 1.0f, true));
}

__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float x) {
  uint32_t u = f2u(x);
  uint32_t s = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return s | 0x7fu;                  // NaN
  if (a >= 0x43e00000u) return s | 0x7eu;                 // |x| >= 448 (and inf): saturate
  if (a < 0x3c800000u) {                                  // below 2^-6: multiples of 2^-9
    float v = __builtin_rintf(u2f(a) * 512.0f);           // exact scaling, then round-half-even
    return s | (uint32_t)v;                               // 8 -> code 0x08 = 2^-6, as wanted
  }
  uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
  return s | (r - 960u);                                  // rebias exponent 127 -> 7
}

// ---- stochastic rounding ------------------------------------------------------------------------
// gfx950's v_cvt_sr_bf16_f32 / v_cvt_sr_fp8_f32, fed the 16 random bits in the upper half of the
// random operand, implement exactly the rule above (checked over all 2^16 random values on finite
// inputs, subnormals included). The FP8 instruction turns |t| >= 448 into NaN rather than
// saturating, so the input is clamped first; a NaN input gives a NaN code.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// BF16 SR of t into the low (hi = false) or high half of `old`; rhi holds the random bits in 31..16
__device__ __forceinline__ uint32_t sr_bf16_into(uint32_t old, float t, uint32_t rhi, bool hi) {
  bf16x2_t o = __builtin_bit_cast(bf16x2_t, old);
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_sr_bf16_f32(o, t, rhi, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_sr_bf16_f32(o, t, rhi, false));
}

// NaN-propagating (IEEE 754-2019 maximum / minimum: v_maximum3_f32, v_minimum3_f32)
__device__ __forceinline__ float clamp_e4m3(float t) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(t, -448.0f), 448.0f);
}

// E4M3 SR of t into byte `sel` of `old`; rhi holds the random bits in 31..16
template <int SEL>
__device__ __forceinline__ uint32_t sr_e4m3_into(uint32_t old, float t, uint32_t rhi) {
  return (uint32_t)__builtin_amdgcn_cvt_sr_fp8_f32(clamp_e4m3(t), (int)rhi, (int)old, SEL);
}

__device__ __forceinline__ uint32_t sr_bf16(float t, uint32_t r16) { return sr_bf16_into(0u, t, r16 << 16, false) & 0xffffu; }
__device__ __forceinline__ uint32_t sr_e4m3(float t, uint32_t r16) { return sr_e4m3_into<0>(0u, t, r16 << 16) & 0xffu; }

// ---- MX-scaled FP4 (OCP Microscaling: 32 E2M1 elements share one E8M0 scale) -------------------
// E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7, bit 3 the sign); E8M0 code c is 2^(c - 127).
// Stochastic rounding of t / scale (scale = 2^X, X in [-127, 127]) to E2M1 with the 16 random
// bits r: the spacing u of the E2M1 grid is 0.5 below 2, 1 below 4 and 2 below 6 (magnitudes of 6
// and above saturate to 6); the magnitude in units of u splits into its floor n and fraction f, and
// it rounds up iff floor(f * 2^16) + r >= 2^16 (the rule of the BF16 and E4M3 roundings). gfx950's
// scaled FP4 conversion with stochastic rounding computes exactly this for the first value of its
// pair when r sits in bits 31..16 of its random operand and bits 15..0 are zero (checked on the
// device against the rule over every range of the grid, signed zeros, subnormal inputs, infinities
// and scales 2^-127 .. 2^127); the pair's second value (here +0, code 0) would take the operand
// shifted left by one bit, so one conversion serves one element. Only the low nibble of the result
// is defined here. rhi: the draw in bits 31..16. Returns the 4-bit code.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t sr_e2m1_scaled(float t, float scale, uint32_t rhi) {
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2_t{t, 0.0f}, rhi, scale, 0) & 15u;
}

// the block exponent X = clamp(floor(log2 amax) - 2, -127, 127) for a finite amax > 0 (v_frexp_exp:
// amax = m 2^e with m in [0.5, 1), so floor(log2 amax) = e - 1); 0 gives -127 and infinity 127
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  if (amax == __builtin_inff()) return 127;
  const int x = __builtin_amdgcn_frexp_expf(amax) - 3;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// two E2M1 codes (byte `sel` of w) times the E8M0 scale c as a BF16 pair (gfx950's scaled FP4 ->
// BF16 conversion: exact for the scales that keep the products inside BF16's range)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  c &= 0xffu;
  return c == 0u ? u2f(0x00400000u) : (c == 255u ? u2f(0x7fc00000u) : u2f(c << 23));   // 2^-127 is subnormal
}

// ---- Philox4x32-10 ------------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

// a ^ b ^ k in one instruction (gfx950's three-input bitwise op, truth table 0x96 = parity)
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  return (uint32_t)__builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

// one Philox4x32 round with round key (k0, k1) (wave-uniform); round i of the 10 uses the key
// (seed_lo + i * 0x9E3779B9, seed_hi + i * 0xBB67AE85)
__device__ __forceinline__ u32x4 philox_round(u32x4 c, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)c.x * 0xD2511F53u, p1 = (uint64_t)c.z * 0xCD9E8D57u;
  return u32x4{xor3_key((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
               xor3_key((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0};
}

// the same round applied to two counters. Inside a large kernel the compiler splits each 32 x 32
// -> 64-bit product into v_mul_lo_u32 + v_mul_hi_u32; the four products are written here as
// v_mad_u64_u32 in one block (their carry-out is unused and shares one SGPR pair, as in the
// compiler's own code for such products), so that no hazard padding separates them.
__device__ __forceinline__ void philox_round2(u32x4& a, u32x4& b, uint32_t k0, uint32_t k1) {
  uint64_t pa0, pa1, pb0, pb1, cy;
  asm("v_mad_u64_u32 %0, %4, %5, %9, 0\n\t"
      "v_mad_u64_u32 %1, %4, %6, %10, 0\n\t"
      "v_mad_u64_u32 %2, %4, %7, %9, 0\n\t"
      "v_mad_u64_u32 %3, %4, %8, %10, 0"
      : "=&v"(pa0), "=&v"(pa1), "=&v"(pb0), "=&v"(pb1), "=&s"(cy)
      : "v"(a.x), "v"(a.z), "v"(b.x), "v"(b.z), "s"(0xD2511F53u), "s"(0xCD9E8D57u));
  a = u32x4{xor3_key((uint32_t)(pa1 >> 32), a.y, k0), (uint32_t)pa1, xor3_key((uint32_t)(pa0 >> 32), a.w, k1), (uint32_t)pa0};
  b = u32x4{xor3_key((uint32_t)(pb1 >> 32), b.y, k0), (uint32_t)pb1, xor3_key((uint32_t)(pb0 >> 32), b.w, k1), (uint32_t)pb0};
}
__device__ __forceinline__ uint32_t philox_key0(uint64_t seed, int i) { return (uint32_t)seed + (uint32_t)i * 0x9E3779B9u; }
__device__ __forceinline__ uint32_t philox_key1(uint64_t seed, int i) { return (uint32_t)(seed >> 32) + (uint32_t)i * 0xBB67AE85u; }

// the counter of element block g at `step`
__device__ __forceinline__ u32x4 philox_counter(uint64_t g, uint64_t step) {
  return u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint64_t seed) {
#pragma unroll
  for (int i = 0; i < 10; ++i) c = philox_round(c, philox_key0(seed, i), philox_key1(seed, i));
  return c;
}

// The 8 random 16-bit values of element block g (the element indices 8g .. 8g + 7), packed two per
// word: position p = idx & 7 takes 16-bit half p & 1 of word p >> 1 (seed wave-uniform).
__device__ __forceinline__ u32x4 rng_block(uint64_t seed, uint64_t step, uint64_t g) {
  return philox4x32_10(philox_counter(g, step), seed);
}

__device__ __forceinline__ uint32_t rng_pick(const u32x4& r, int e) {   // e = position p
  uint32_t w = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// the 16 random bits of element idx
__device__ __forceinline__ uint32_t rng_r16(uint64_t seed, uint64_t step, uint64_t idx) {
  return rng_pick(rng_block(seed, step, idx >> 3), (int)(idx & 7));
}

// the same 16 bits placed in bits 31..16 (the form the SR instructions take)
__device__ __forceinline__ uint32_t rng_pick_hi(const u32x4& r, int e) {
  uint32_t w = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
  return (e & 1) ? (w & 0xffff0000u) : (w << 16);
}

// ---- sigmoid-BCE gradient -----------------------------------------------------------------------
// g = sigmoid(z) - y = s / (1 + e^a) with a = -z, s = 1 (y = 0) or a = z, s = -1 (y = 1): the
// cancellation-free forms. e^a = 2^(a log2 e) with the product carried to ~48 bits so that its
// rounding does not reach the result, v_exp_f32, one correction of the exponent's low part, then
// v_rcp_f32: about 3 FP32 ulp overall, some 2^-15 of a BF16 unit, so the BF16 gradient code
// differs from the correctly rounded one only for values that close to a rounding boundary.
// Where the reciprocal leaves the normal range (|z| > 80) the exact-division form is used.
// the fast form, valid for |z| <= 80, with the label as a sign mask: bit 31 of ys set for y = 1
// (the sign flips of a and of the result are then one bit operation each)
__device__ __forceinline__ float bce_grad_fast_m(float z, uint32_t ys) {
  constexpr float L2E_HI = 1.44269502162933349609375f;         // FP32(log2 e)
  constexpr float LN2 = 0.693147180559945309f;
  constexpr float L2E_LO_LN2 = 1.33498838e-08f;                // (log2 e - L2E_HI) ln 2
  // bitop3 truth tables index (src0, src1, src2) as bits (2, 1, 0): 0xD2 = s0 ^ (~s1 & s2),
  // 0x78 = s0 ^ (s1 & s2)
  const float a = u2f(__builtin_amdgcn_bitop3_b32(f2u(z), ys, 0x80000000u, 0xD2));   // -z (y = 0), z (y = 1)
  const float p = a * L2E_HI;
  const float t = fmaf(a, L2E_HI, -p);                         // exact: a L2E_HI - p
  const float c = fmaf(t, LN2, a * L2E_LO_LN2);                // (a log2 e - p) ln 2
  float e = __builtin_amdgcn_exp2f(p);
  e = fmaf(e, c, e);                                           // e^a = 2^p e^c
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return u2f(__builtin_amdgcn_bitop3_b32(f2u(r), ys, 0x80000000u, 0x78));          // r (y = 0), -r (y = 1)
}

// the small-argument form, for |z| <= 2: 2^(a log2 e) straight from the FP32 product. Its rounding
// (at most 2^-23 in the exponent argument) and that of log2 e add under 1.5 FP32 ulp, so this form
// stays within about 4 ulp of sigmoid, with two operations per element fewer than the split form.
__device__ __forceinline__ float bce_grad_small_m(float z, uint32_t ys) {
  constexpr float L2E_HI = 1.44269502162933349609375f;         // FP32(log2 e)
  const float a = u2f(__builtin_amdgcn_bitop3_b32(f2u(z), ys, 0x80000000u, 0xD2));
  const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * L2E_HI));
  return u2f(__builtin_amdgcn_bitop3_b32(f2u(r), ys, 0x80000000u, 0x78));
}

// the same two forms for y = 0, g = sigmoid(z), with a = -z taken by the operations' sign
// modifiers (bit-identical to the forms above with the label mask 0)
__device__ __forceinline__ float bce_grad_fast_y0(float z) {
  constexpr float L2E_HI = 1.44269502162933349609375f;
  constexpr float LN2 = 0.693147180559945309f;
  constexpr float L2E_LO_LN2 = 1.33498838e-08f;
  const float a = -z;
  const float p = a * L2E_HI;
  const float t = fmaf(a, L2E_HI, -p);
  const float c = fmaf(t, LN2, a * L2E_LO_LN2);
  float e = __builtin_amdgcn_exp2f(p);
  e = fmaf(e, c, e);
  return __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float bce_grad_small_y0(float z) {
  constexpr float L2E_HI = 1.44269502162933349609375f;
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * L2E_HI));
}

__device__ __forceinline__ float bce_grad_fast(float z, bool y) { return bce_grad_fast_m(z, y ? 0x80000000u : 0u); }

// the exact-division form, for |z| > 80
__device__ __forceinline__ float bce_grad_slow(float z, bool y) {
  const float r = 1.0f / (1.0f + expf(y ? z : -z));
  return y ? -r : r;
}

__device__ __forceinline__ float bce_grad(float z, bool y) {
  if (__builtin_expect(__builtin_fabsf(z) > 80.0f, 0)) return bce_grad_slow(z, y);
  if (__builtin_fabsf(z) <= 2.0f) return bce_grad_small_m(z, y ? 0x80000000u : 0u);
  return bce_grad_fast(z, y);
}

// summed-loss term: max(z, 0) - y z + log1p(e^-|z|)
__device__ __forceinline__ float bce_loss(float z, bool y) {
  return fmaxf(z, 0.0f) - (y ? z : 0.0f) + log1pf(expf(-fabsf(z)));
}

}  // namespace elmo
