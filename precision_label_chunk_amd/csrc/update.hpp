// The fused SGD update with stochastic rounding straight from a wave's 32 x 32 dW accumulator
// block, and the LDS row swizzle of the weight and gradient tiles it reads. Shared by the two-kernel
// backward (step_chunks.hip) and the single-pass step (step_single.hip).
//
// Method: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large Output Spaces"
// (summary page, "Approach": momentum-free SGD fused with the classifier gradient, stochastic
// rounding of pure BF16/FP8 weights; "Limitations": FP4 weights with micro-tensor scaling).
#pragma once
#include "mfma.hpp"
#include "numerics.hpp"
#include "step_kernels.hpp"

namespace elmo {

// LDS tiles keep rows of CPR 16-byte chunks; chunk c of row j sits at slot c ^ row_swz<CPR>(j).
// gfx950's LDS has 64 four-byte banks: ds_read_b128 serves 16 lanes per cycle, ds_read_b64 and
// ds_read_b64_tr_b16 32 lanes, so a read is conflict-free when each such lane group covers 256
// distinct bytes modulo 256. The swizzle makes that hold for the two read shapes used below:
// one chunk of 16 consecutive rows (ds_read_b128), and 4 consecutive chunks of 4 consecutive rows
// (the 32-lane view of a transposing read), for rows of 512/256 bytes (a 4-bit XOR), 128 bytes
// (2 rows per bank window) and 64 bytes (4 rows per window).
template <int CPR>
__device__ __forceinline__ int row_swz(int j) {
  const int j0 = j & 1, j1 = (j >> 1) & 1, j2 = (j >> 2) & 1, j3 = (j >> 3) & 1;
  if constexpr (CPR >= 16) return j2 | (j0 << 1) | (j1 << 2) | ((j0 ^ j3) << 3);
  else if constexpr (CPR == 8) return j2 | (j3 << 1) | (j1 << 2);
  else return j2 | (j3 << 1);
}

// The fused SGD step with stochastic rounding for one wave's 32 labels x 32 features, straight
// from its dW accumulators. Lane (l32, hi) holds label l32 and, in register 8u + p (u = 0, 1,
// p = 0..7), feature 16u + 8 (p >> 2) + 4 hi + (p & 3) of the 32. The 32 features are the RNG
// blocks 4 grp .. 4 grp + 3 (eight consecutive features each, grp the index of the row's 32-element
// group), and register 8u + p sits in block 4 grp + 2u + (p >> 2) at position 4 hi + (p & 3): a
// lane holds half of each of the four blocks. Lane half hi computes the two blocks 4 grp + 2 hi and
// + 1 (Philox rounds on both at once), then the lane pair swaps the halves of the output words each
// side needs (four v_permlane32_swap): afterwards words 2k + w (k, w = 0, 1) of u32x4 R_u hold word
// 2 hi + w of block 4 grp + 2u + k, so that register 8u + p takes 16-bit half p & 1 of word p >> 1 of
// R_u. Then t = fmaf(-lr, dW, w) and hardware stochastic rounding per element. Swapping the packed
// results of u = 1 of lane half 0 with those of u = 0 of lane half 1 leaves each lane the 16
// consecutive features 16 hi .. 16 hi + 15 of its label, stored in 16-byte pieces. The work is cut
// into UPD_PHASES phases so that it can be spread between MFMAs: 0 the RNG counters, 1..10 the
// Philox rounds and after the last the word exchange (these RNG_PHASES need no dW), 11 old-weight
// reads, 12..19 two weights each (rounding and packing), 20 the exchange and the stores.
//   ow    the label's W row in the LDS tile (BF16); owa/owb[u] element offsets of the runs
//         16u + 4 hi and 16u + 8 + 4 hi of the wave's features in it
//   roff  byte offset of the label's row in the chunk's weight resource plus that of the wave's
//         first feature
//   grp   (global element index of the wave's first feature in the label's row) >> 5
constexpr int UPD_PHASES = 21, RNG_PHASES = 11;
struct UpdState {
  u32x4 c[2];
  i32x4_t ow[2];
  uint32_t pk[8];                              // packed results: 4 words per block (BF16), 2 (E4M3)
  uint32_t amax;                               // MXFP4: largest |t| (bit pattern; NaN above +inf)
  float scale;                                 // MXFP4: the block's scale 2^X (NaN: a NaN block)
};

// MXFP4 (the 32 features are one scale block): phases 12..15 compute four values t each and the
// lane's largest magnitude, 16 takes the block's from the lane pair and its shared exponent X,
// 17..20 recompute four values t each (re-reading the old weights from LDS: cheaper than keeping
// all 16 values or their weights live) and round
// t / 2^X to E2M1 (the hardware's scaled conversion, one element each), packing runs of four codes
// (16 bits); then the lane pair swaps halves so that
// lane half hi holds bytes 8 hi .. 8 hi + 7 of the block's 16 code bytes, and lane half 0 also
// stores the scale byte (at soff).
template <int WF>
__device__ __forceinline__ void upd_phase_mx(int p, UpdState& st, const f32x16_t& acc, const uint16_t* ow,
                                             const int (&owa)[2], const int (&owb)[2], __amdgpu_buffer_rsrc_t wres,
                                             int roff, int soff, int hi, float lr) {
  auto tval = [&](int u, int hf, int e) {                      // register 8u + 4 hf + e
    const uint32_t wb = (uint32_t)st.ow[u][2 * hf + (e >> 1)];
    return fmaf(-lr, acc[8 * u + 4 * hf + e], u2f((e & 1) ? (wb & 0xffff0000u) : (wb << 16)));
  };
  if (p < 16) {
    const int u = (p - 12) >> 1, hf = (p - 12) & 1;
    if (p == 12) st.amax = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t m = f2u(tval(u, hf, e)) & 0x7fffffffu;
      st.amax = m > st.amax ? m : st.amax;
    }
  } else if (p == 16) {
    const auto sw = __builtin_amdgcn_permlane32_swap(st.amax, st.amax, false, false);
    const uint32_t m = (uint32_t)sw[0] > (uint32_t)sw[1] ? (uint32_t)sw[0] : (uint32_t)sw[1];
    // 2^X, or NaN for a block with a NaN (scale code 255); its E8M0 code is its bits >> 23 (2^-127,
    // the one subnormal scale, is 0x00400000: code 0)
    st.scale = e8m0_to_f32(m > 0x7f800000u ? 255u : (uint32_t)(mx_block_exponent(u2f(m)) + 127));
  } else {
    const int u = (p - 17) >> 1, hf = (p - 17) & 1;
    if (hf == 0) {
      // the old weights of block u again from the LDS tile (shorter register lifetimes than
      // keeping all of them from phase 11)
      const i32x2_t a = *(const i32x2_t*)(ow + owa[u]), b = *(const i32x2_t*)(ow + owb[u]);
      st.ow[u] = i32x4_t{a[0], a[1], b[0], b[1]};
    }
    uint32_t run = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      run |= sr_e2m1_scaled(tval(u, hf, e), st.scale, rng_pick_hi(st.c[u], 4 * hf + e)) << (4 * e);
    st.pk[2 * u + hf] = st.scale != st.scale ? 0u : run;
    if (p == 20) {
      // runs 4u + 2 hf + hi of the block; A = runs hi | 2 + hi, B = runs 4 + hi | 6 + hi
      const auto sw = __builtin_amdgcn_permlane32_swap(st.pk[0] | (st.pk[1] << 16), st.pk[2] | (st.pk[3] << 16),
                                                       false, false);
      const uint32_t x = (uint32_t)sw[0], y = (uint32_t)sw[1];
      const i32x2_t v = {(int)((x & 0xffffu) | (y << 16)), (int)((x >> 16) | (y & 0xffff0000u))};
      __builtin_amdgcn_raw_buffer_store_b64(v, wres, roff + 8 * hi, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(f2u(st.scale) >> 23), wres, hi == 0 ? soff : 0x7ffffff0, 0, 0);
    }
  }
}

template <int WF>
__device__ __forceinline__ void upd_phase(int p, UpdState& st, const f32x16_t& acc, const uint16_t* ow,
                                          const int (&owa)[2], const int (&owb)[2], __amdgpu_buffer_rsrc_t wres,
                                          int roff, int soff, uint64_t grp, int hi, float lr, uint64_t seed,
                                          uint64_t step) {
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
  if constexpr (WF == W_MXFP4_) {
    if (p >= 12) {
      upd_phase_mx<WF>(p, st, acc, ow, owa, owb, wres, roff, soff, hi, lr);
      sched_fence();                           // (keeps the phases' register lifetimes apart)
      return;
    }
  }
  if (p == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) st.c[k] = philox_counter(4 * grp + 2 * hi + k, step);
  } else if (p <= 10) {
    const uint32_t k0 = philox_key0(seed, p - 1), k1 = philox_key1(seed, p - 1);
    philox_round2(st.c[0], st.c[1], k0, k1);
    if (p == 10) {
      // word w of lane half 1's blocks (4 grp + 2 + k) <-> word 2 + w of lane half 0's blocks
      // (4 grp + k): each side keeps its own half of the words and receives the other's
      const auto s00 = __builtin_amdgcn_permlane32_swap(st.c[0].x, st.c[0].z, false, false);
      const auto s01 = __builtin_amdgcn_permlane32_swap(st.c[0].y, st.c[0].w, false, false);
      const auto s10 = __builtin_amdgcn_permlane32_swap(st.c[1].x, st.c[1].z, false, false);
      const auto s11 = __builtin_amdgcn_permlane32_swap(st.c[1].y, st.c[1].w, false, false);
      st.c[0] = u32x4{(uint32_t)s00[0], (uint32_t)s01[0], (uint32_t)s10[0], (uint32_t)s11[0]};
      st.c[1] = u32x4{(uint32_t)s00[1], (uint32_t)s01[1], (uint32_t)s10[1], (uint32_t)s11[1]};
    }
  } else if (p == 11) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const i32x2_t a = *(const i32x2_t*)(ow + owa[u]), b = *(const i32x2_t*)(ow + owb[u]);
      st.ow[u] = i32x4_t{a[0], a[1], b[0], b[1]};
    }
  } else if (p < 20) {
    const int u = (p - 12) >> 2, pr = (p - 12) & 3;          // positions 2 pr, 2 pr + 1 of block u
    const u32x4& rnd = st.c[u];
    const uint32_t wb = (uint32_t)st.ow[u][pr];
    const float t0 = fmaf(-lr, acc[8 * u + 2 * pr], u2f(wb << 16));
    const float t1 = fmaf(-lr, acc[8 * u + 2 * pr + 1], u2f(wb & 0xffff0000u));
    if constexpr (WF == W_BF16_) {
      // (the BF16 rounding uses bits 31..16 of its random operand only: the odd position takes its
      // word as it is)
      const uint32_t w = (pr >> 1) == 0 ? ((pr & 1) ? rnd.y : rnd.x) : ((pr & 1) ? rnd.w : rnd.z);
      const uint32_t lo = sr_bf16_into(0u, t0, w << 16, false);
      st.pk[4 * u + pr] = sr_bf16_into(lo, t1, w, true);
    } else {
      // bytes 2 (pr & 1), 2 (pr & 1) + 1 of the word of run pr >> 1
      uint32_t o = (pr & 1) ? st.pk[2 * u + (pr >> 1)] : 0u;
      if (pr & 1) {
        o = sr_e4m3_into<2>(o, t0, rng_pick_hi(rnd, 2 * pr));
        o = sr_e4m3_into<3>(o, t1, rng_pick_hi(rnd, 2 * pr + 1));
      } else {
        o = sr_e4m3_into<0>(o, t0, rng_pick_hi(rnd, 2 * pr));
        o = sr_e4m3_into<1>(o, t1, rng_pick_hi(rnd, 2 * pr + 1));
      }
      st.pk[2 * u + (pr >> 1)] = o;
    }
  } else {
    // word k of block 0 (lane half 1) <-> word k of block 1 (lane half 0): then words x (own) and
    // y (received) of each run are features 16 hi + 8 run + 0..3 and + 4..7
    constexpr int NW = WF == W_BF16_ ? 4 : 2;
    uint32_t x[NW], y[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const auto sw = __builtin_amdgcn_permlane32_swap(st.pk[k], st.pk[NW + k], false, false);
      x[k] = (uint32_t)sw[0];
      y[k] = (uint32_t)sw[1];
    }
    const int off = roff + 16 * hi * ESZ;
    if constexpr (WF == W_BF16_) {
      buffer_store16(i32x4_t{(int)x[0], (int)x[1], (int)y[0], (int)y[1]}, wres, off);
      buffer_store16(i32x4_t{(int)x[2], (int)x[3], (int)y[2], (int)y[3]}, wres, off + 16);
    } else {
      buffer_store16(i32x4_t{(int)x[0], (int)y[0], (int)x[1], (int)y[1]}, wres, off);
    }
  }
}

}  // namespace elmo
