// The MX-scaled FP4 logit tile on the scaled matrix cores, shared by the training forward and the
// top-k scan: one wave's MI x NI blocks of 32 x 32 logits Z = X~ W^T, E4M3 features (block scale 1)
// times E2M1 weights with their E8M0 scales, one 32 x 32 x 64 MFMA per K step and block. Each lane
// loads its own operand fragments with buffer loads, one K step ahead of their use: rows past a
// resource's end read as zero.
//   xres  the E4M3 feature rows (D bytes each); the wave's rows start at xrow0
//   wres  MXFP4 weight rows (D/2 code bytes, D/32 scale bytes: rb bytes); the wave's at wrow0
// With D % 256 == 0 the rows (17 D / 32 bytes) are 8-byte aligned, so the code fragments are read
// in 8-byte pieces.
#pragma once
#include "mfma.hpp"

namespace elmo {

template <int MI, int NI>
__device__ __forceinline__ void mx_logit_tile(f32x16_t (&acc)[MI][NI], __amdgpu_buffer_rsrc_t xres, int xrow0, int D,
                                              __amdgpu_buffer_rsrc_t wres, int wrow0, int rb, int l32, int hi) {
  const int nk = D / 64;
  // K step kk: A = feature row xrow0 + 32 mi + l32, bytes kk 64 + 16 hi .. +15 and kk 64 + 32 + 16 hi
  // .. +15 (the E4M3 operand's K order beside an FP4 one); B = weight row wrow0 + 32 ni + l32, code
  // bytes kk 32 + 16 hi .. +15 and the scale byte of block 2 kk + hi
  struct Frag { i32x8_t a[MI]; i32x4_t b[NI]; int sc[NI]; };
  auto load = [&](int kk, Frag& f) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int o = (xrow0 + 32 * mi + l32) * D + kk * 64 + hi * 16;
      const i32x4_t a0 = buffer_load16(xres, o), a1 = buffer_load16(xres, o + 32);
      f.a[mi] = i32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = wrow0 + 32 * ni + l32;
      const i32x2_t b0 = __builtin_amdgcn_raw_buffer_load_b64(wres, row * rb + kk * 32 + hi * 16, 0, 0);
      const i32x2_t b1 = __builtin_amdgcn_raw_buffer_load_b64(wres, row * rb + kk * 32 + hi * 16 + 8, 0, 0);
      f.b[ni] = i32x4_t{b0[0], b0[1], b1[0], b1[1]};
      f.sc[ni] = (int)__builtin_amdgcn_raw_buffer_load_b8(wres, row * rb + D / 2 + 2 * kk + hi, 0, 0);
    }
  };
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
  Frag cur, nxt;
  load(0, cur);
  for (int kk = 0; kk < nk; ++kk) {
    if (kk + 1 < nk) load(kk + 1, nxt);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const i32x8_t bv = {cur.b[ni][0], cur.b[ni][1], cur.b[ni][2], cur.b[ni][3], 0, 0, 0, 0};
        acc[mi][ni] = mfma_e4m3_fp4(cur.a[mi], bv, acc[mi][ni], 127, cur.sc[ni]);
      }
    cur = nxt;
  }
}

}  // namespace elmo
