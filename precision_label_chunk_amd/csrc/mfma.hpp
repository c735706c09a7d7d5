// CDNA4 (gfx950) matrix-core and LDS helpers.
//
// Operand layouts (checked on the device with exact-integer inputs):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row m = l%32, k = 8*(l/32) + e, e = 0..7
//                             B: lane l holds col n = l%32, k = 8*(l/32) + e
//                             C: lane l, register i holds col n = l%32, row m = 8*(i/4) + 4*(l/32) + i%4
//   v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, no block scaling): as above with k = 32*(l/32) + e,
//                             e = 0..31 bytes; it reads 0x7E as 448 and honours subnormals.
//                             (With both operands 8-bit only their common K order matters.)
//   v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 A x E2M1 B: B lane l holds col n = l%32, k = 32*(l/32) + e,
//                             e = 0..31 in 16 bytes (element e in nibble e & 1 of byte e / 2); A lane l
//                             holds row m = l%32 with k = 16*(l/32) + e in bytes 0..15 and
//                             k = 32 + 16*(l/32) + e - 16 in bytes 16..31; each lane's E8M0 scale
//                             (byte 0 of the operand) applies to its row's / column's K block
//                             [32*(l/32), 32*(l/32) + 32).
//   ds_read_b64_tr_b16        a group of 16 lanes reads a 4 x 16 block of 16-bit elements whose
//                             row r is supplied (4 consecutive elements each) by lanes 4r..4r+3;
//                             lane i of the group receives column i (rows 0..3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace elmo {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x16_t mfma_bf16(s16x8_t a, s16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_e4m3(i32x8_t a, i32x8_t b, f32x16_t c) {
  // format 0 = E4M3 for both operands; zero scale operands select the unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// E4M3 A x E2M1 B with E8M0 block scales (one per lane: the scale of its 32-element K block; the
// FP4 operand takes the low four registers)
__device__ __forceinline__ f32x16_t mfma_e4m3_fp4(i32x8_t a, i32x8_t b, f32x16_t c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, scale_b);
}

// the same with the B operand's four code dwords and its scale taken from byte OPSEL_B of scale_b
// (the A operand's scale 1.0)
template <int OPSEL_B>
__device__ __forceinline__ f32x16_t mfma_e4m3_fp4_sel(i32x8_t a, i32x4_t b, f32x16_t c, int scale_b) {
  const i32x8_t bv = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bv, c, 0, 4, 0, 127, OPSEL_B, scale_b);
}

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// p must point into __shared__ memory and be 8-byte aligned
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<uint16_t*>(p)));
}

// Raw buffer access through a resource of `bytes` bytes at `base` (both wave-uniform): loads at or
// beyond the end return zeros and stores there are dropped by the hardware's range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ i32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// with a wave-uniform byte offset added (the instruction's scalar offset)
__device__ __forceinline__ i32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int off, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
}
__device__ __forceinline__ void buffer_store16(i32x4_t v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// f(std::integral_constant<int, I>) for I = B .. E-1, expanded at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// no instruction is scheduled across this point
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ s16x8_t join(s16x4_t lo, s16x4_t hi) {
  return s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace elmo
