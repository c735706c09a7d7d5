// The forward contraction of one (all-samples x 128-label) tile on the matrix cores, shared by the
// training step's forward kernel and the top-k scoring kernel:
//   acc[b][j] = sum_k Xf[b][k] * W[j][k]
// with Xf the zero-padded feature rows (BF16, or E4M3 for E4M3 weights) and W the tile's weight
// rows (rows at or beyond `nvalid` read as zero). Operands are staged through LDS in 128-byte K
// slices, double buffered, with the next slice's global loads in flight during this slice's MFMAs.
#pragma once
#include "mfma.hpp"
#include "step_kernels.hpp"

namespace elmo {

constexpr int fwd_smem_bytes(int MB) { return 2 * (MB + TJ1) * P1; }

// RW x CW is this wave's sub-tile (RW samples, CW labels); the work-group is (MB/RW) x (TJ1/CW) waves
template <int MB, int WF, int RW, int CW>
__device__ __forceinline__ void fwd_tile(f32x16_t (&acc)[RW / 32][CW / 32], uint8_t* smem,
                                         const uint8_t* __restrict__ Wt, int nvalid,
                                         const uint8_t* __restrict__ Xf, int64_t rowbytes, int tid, int wb,
                                         int wj) {
  constexpr int MI = RW / 32, NI = CW / 32;
  constexpr int SLICE = (MB + TJ1) * P1;
  constexpr int CPT = (MB + TJ1) * (KSB / 16) / 256;
  static_assert((MB + TJ1) * (KSB / 16) % 256 == 0, "slice split");
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int nks = (int)((rowbytes + KSB - 1) / KSB);

  i32x4_t stg[CPT];
  auto gload = [&](int ks) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * 256, row = ci >> 3, part = ci & 7;
      const int64_t boff = (int64_t)ks * KSB + part * 16;
      i32x4_t v = {0, 0, 0, 0};
      if (boff < rowbytes) {
        if (row < MB) v = *(const i32x4_t*)(Xf + row * rowbytes + boff);
        else if (row - MB < nvalid) v = *(const i32x4_t*)(Wt + (int64_t)(row - MB) * rowbytes + boff);
      }
      stg[c] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * 256, row = ci >> 3, part = ci & 7;
      *(i32x4_t*)(smem + buf * SLICE + row * P1 + part * 16) = stg[c];
    }
  };

#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload(ks + 1);
    const uint8_t* Xs = smem + buf * SLICE;
    const uint8_t* Ws = Xs + MB * P1;
    if constexpr (WF == W_BF16_) {
#pragma unroll
      for (int kk = 0; kk < KSB / 32; ++kk) {
        s16x8_t a[MI], b[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) a[mi] = *(const s16x8_t*)(Xs + (wb * RW + mi * 32 + l32) * P1 + kk * 32 + hi * 16);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) b[ni] = *(const s16x8_t*)(Ws + (wj * CW + ni * 32 + l32) * P1 + kk * 32 + hi * 16);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma_bf16(a[mi], b[ni], acc[mi][ni]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSB / 64; ++kk) {
        i32x8_t a[MI], b[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const uint8_t* p = Xs + (wb * RW + mi * 32 + l32) * P1 + kk * 64 + hi * 32;
          const i32x4_t x0 = *(const i32x4_t*)p, x1 = *(const i32x4_t*)(p + 16);
          a[mi] = i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const uint8_t* p = Ws + (wj * CW + ni * 32 + l32) * P1 + kk * 64 + hi * 32;
          const i32x4_t x0 = *(const i32x4_t*)p, x1 = *(const i32x4_t*)(p + 16);
          b[ni] = i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma_e4m3(a[mi], b[ni], acc[mi][ni]);
      }
    }
    if (ks + 1 < nks) lstore(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace elmo
