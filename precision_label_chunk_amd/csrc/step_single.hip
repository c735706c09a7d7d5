// The single-pass variant of the chunked, fused XMC classifier-head step on gfx950: one kernel per
// label chunk that computes each weight tile's logits, gradient, input-gradient contribution and
// stochastic-rounding SGD update while the tile sits in LDS, for padded batches of 32 samples
// (B <= 32) and D = 256, 512 or 768. The gradient never leaves the compute unit, the weights are
// read once and written once per step, and no chunk-sized transient is written at all.
//
// Method: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large Output Spaces"
// (summary page, "Approach": the classifier gradient computation fused with the SGD update, pure
// BF16/FP8 weights with stochastic rounding, the label dimension chunked; arXiv abstract:
// "gradient fusion and chunking").
//
// Why only B <= 32: the input gradient dX = G W_old reduces over every label into a B x D FP32
// accumulator. A work-group that owns whole weight rows (which the logits need) can keep that
// accumulator in registers for the whole launch only while B x D x 4 bytes, the stationary
// features in both fragment orders and the dW accumulators of one 32 x 32 block per wave fit beside
// the update's own state: at D = 768 that is 96 KiB + 2 x 48 KiB + 32 KiB of the 512 KiB register
// file at 32 samples (243-247 of a wave's 256 registers in use), and the first three double at 64
// samples. Wider batches keep the two-kernel step of step_chunks.hip.
//
// Work-group (one per CU, 8 waves, a contiguous range of the chunk's 32-label tiles): wave w owns
// features [32 NFW w, 32 NFW (w + 1)) (NFW = D / 256 feature blocks of 32). Per tile:
//   1. Z partial: the wave's D / 128 K steps of Z[32 samples][32 labels] = X~ W_t^T (BF16 MFMA;
//      A = its features of X~ stationary in registers, B = the tile's rows from LDS), stored to LDS;
//   2. wave w sums the eight partials of accumulator registers 2w, 2w + 1 in a fixed order (the
//      logits of samples 8 (w >> 1) + 4 hi + 2 (w & 1) + {0, 1} of label l32) and forms
//      G = BF16_RNE(sigmoid(Z) - Y) into the LDS G tile (label-major [32][32]);
//   3. dW^T[d][j] = sum_b X^T[d][b] G[b][j] over the wave's NFW feature blocks (A = stationary X^T
//      fragments, B = G rows) and dX^T[d][b] += sum_j W_t^T[d][j] G^T[j][b] (A = W^T, B = G^T, both
//      transposing LDS reads); the dX^T accumulators live in registers for the whole launch;
//   4. the next tile, loaded into registers at the start of the iteration, is decoded to BF16 into
//      the other LDS buffer, and its positives gathered into label bits;
//   5. the update of the wave's 32 x 32 blocks from the dW accumulators (the same code as the
//      two-kernel backward: Philox draws, fmaf, hardware SR), stored in place.
// Three barriers per tile. At the end each work-group stores its dX^T accumulators as its range's
// running partial (the two-kernel step's partial layout), which the step's fixed-order reduction
// sums. X~ is X for BF16 weights and E4M3-RNE(X) for E4M3 and MXFP4 weights, decoded to BF16
// (exact), and the weights are decoded to BF16 in LDS (exact), so the forward runs on the BF16
// matrix cores with the same products as the FP8 and scaled-FP4 forwards.
#include "step_kernels.hpp"

#include <type_traits>

#include "mfma.hpp"
#include "numerics.hpp"
#include "update.hpp"

namespace elmo {

constexpr int SP_TJ = 32;        // labels per tile
constexpr int SP_MB = 32;        // padded samples

template <int WF, int NFW, bool LOSS>
__global__ __launch_bounds__(512, 1) void k_step_single(uint8_t* __restrict__ W, int64_t c0, int clen,
                                                        const uint16_t* __restrict__ Xb,
                                                        const uint8_t* __restrict__ Xq,
                                                        const uint16_t* __restrict__ XbT,
                                                        const uint32_t* __restrict__ tile_off,
                                                        const uint32_t* __restrict__ bucket, int64_t bucket_cap,
                                                        int B, float* __restrict__ part, float lr, uint64_t seed,
                                                        uint64_t step, int first, float* __restrict__ loss_part,
                                                        uint16_t* __restrict__ gout, int64_t gpitch) {
  constexpr int D = 256 * NFW, MB = SP_MB, TJ = SP_TJ;
  constexpr int NKW = 2 * NFW;                 // forward K steps (16 features) per wave
  constexpr int CPR = D / 8;                   // 16-byte chunks per decoded (BF16) LDS row
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
  constexpr int RB = (int)w_row_bytes(WF, D);
  // staging items per tile row: 16-byte chunks (BF16, E4M3) or 16-element parts (MXFP4: 8 code bytes)
  constexpr int WCPR = WF == W_MXFP4_ ? D / 16 : D * ESZ / 16;
  constexpr int WPT = TJ * WCPR / 512;         // staging items per thread
  static_assert(WPT * 512 == TJ * WCPR, "whole staging items per thread");
  __shared__ __attribute__((aligned(1024))) uint16_t Ws[2][TJ * D];
  __shared__ __attribute__((aligned(1024))) f32x4_t Zs[8][4][64];
  __shared__ __attribute__((aligned(1024))) uint16_t Gs[TJ * MB];
  __shared__ uint32_t ybits[4][TJ];           // bit b of word j: sample b is a positive of label j
  __shared__ float lred[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5, q = lane >> 4, li = lane & 15;
  const int nt = (clen + TJ - 1) / TJ;
  const int r = blockIdx.x, NR = gridDim.x;
  const int t0 = (int)((int64_t)nt * r / NR), t1 = (int)((int64_t)nt * (r + 1) / NR);
  // the chunk's weight rows: rows past its end load as zero and their stores are dropped
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + c0 * (int64_t)RB, clen * RB);

  // stationary operands of this wave's features: forward A fragments (lane: sample l32, features
  // 16 kk + 8 hi .. + 7 of K step kk) from the row-major X~ copy, and the dW A fragments (lane:
  // feature l32 of block fb, samples 16 kk + 8 hi .. + 7) from the fragment-ordered X^T copy
  s16x8_t xf[NKW], xT[NFW][2];
#pragma unroll
  for (int k = 0; k < NKW; ++k) {
    const int f0 = 16 * (NKW * wave + k) + 8 * hi;
    if constexpr (WF == W_BF16_) {
      xf[k] = *(const s16x8_t*)(Xb + l32 * D + f0);
    } else {
      const i32x2_t v = *(const i32x2_t*)(Xq + l32 * D + f0);
      uint32_t b[4];
      e4m3x4_to_bf16x4((uint32_t)v[0], b[0], b[1]);
      e4m3x4_to_bf16x4((uint32_t)v[1], b[2], b[3]);
      xf[k] = __builtin_bit_cast(s16x8_t, i32x4_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3]});
    }
  }
#pragma unroll
  for (int i = 0; i < NFW; ++i)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      xT[i][kk] = *(const s16x8_t*)(XbT + (((NFW * wave + i) * 2 + kk) * 64 + lane) * 8);

  // dX^T accumulators of the wave's feature blocks (one sample block), from this work-group's
  // running partial (zero in the step's first chunk): lane l's registers 4 ig .. 4 ig + 3 of feature
  // block fb at ((fb * 4 + ig) * 64 + l) * 4 within the range's slot
  float* slot = part + (int64_t)r * D * MB + 4 * lane;
  f32x16_t accX[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const f32x4_t o = first ? f32x4_t{} : *(const f32x4_t*)(slot + ((NFW * wave + i) * 4 + ig) * 256);
#pragma unroll
      for (int e = 0; e < 4; ++e) accX[i][4 * ig + e] = o[e];
    }

  // LDS element offsets. Weight tile rows (label j, D BF16) keep chunk c at c ^ row_swz<CPR>(j);
  // the G tile ([32 labels][32 samples] BF16) chunk c at c ^ row_swz<4>(j).
  const int swL = row_swz<CPR>(l32);
  //   forward B (row l32, chunk 2 kk + hi)
  auto offF = [&](int kk) { return l32 * D + (((2 * kk + hi) ^ swL) << 3); };
  //   dW B (G row l32, chunk 2 kk + hi)
  const int gW = row_swz<4>(l32);
  int offW[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) offW[kk] = l32 * MB + (((2 * kk + hi) ^ gW) << 3);
  //   dX (transposing reads): rows jX and jX + 4 of each 16-label K step; A = W^T, features
  //   32 fb + 16 (q & 1) + 4 (li & 3) .. + 3; B = G^T, samples 16 (q & 1) + 4 (li & 3) .. + 3
  const int jX = 8 * (q >> 1) + (li >> 2);
  int offA0[NFW], offA1[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int cA = 4 * (NFW * wave + i) + 2 * (q & 1) + ((li & 3) >> 1);
    offA0[i] = jX * D + ((cA ^ row_swz<CPR>(jX)) << 3) + 4 * (li & 1);
    offA1[i] = (jX + 4) * D + ((cA ^ row_swz<CPR>(jX + 4)) << 3) + 4 * (li & 1);
  }
  const int cB = 2 * (q & 1) + ((li & 3) >> 1);
  const int offB0 = jX * MB + ((cB ^ row_swz<4>(jX)) << 3) + 4 * (li & 1);
  const int offB1 = (jX + 4) * MB + ((cB ^ row_swz<4>(jX + 4)) << 3) + 4 * (li & 1);
  //   update: old weights of row l32, features 32 fb + 16 u + 4 hi (chunk 4 fb + 2 u) and + 8
  //   (chunk 4 fb + 2 u + 1), formed per block below

  // staging of a tile through registers: item ci = tid + 512 c is row ci / WCPR, part ci % WCPR
  i32x4_t stg[WPT];
  auto wload = [&](int t) {
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int ci = tid + 512 * c, jr = ci / WCPR, p = ci % WCPR;
      const int ro = (t * TJ + jr) * RB;
      if constexpr (WF == W_MXFP4_) {
        // 16 codes (8 bytes) and the scale byte of their 32-element block
        const i32x2_t cd = __builtin_amdgcn_raw_buffer_load_b64(wres, ro + p * 8, 0, 0);
        const int sc = (int)__builtin_amdgcn_raw_buffer_load_b8(wres, ro + D / 2 + p / 2, 0, 0);
        stg[c] = i32x4_t{cd[0], cd[1], sc, 0};
      } else {
        stg[c] = buffer_load16(wres, ro + p * 16);
      }
    }
  };
  auto wstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int ci = tid + 512 * c, jr = ci / WCPR, p = ci % WCPR;
      const int sw = row_swz<CPR>(jr);
      uint16_t* row = &Ws[buf][jr * D];
      if constexpr (WF == W_BF16_) {
        *(i32x4_t*)(row + ((p ^ sw) << 3)) = stg[c];
      } else if constexpr (WF == W_MXFP4_) {
        const float sc = e8m0_to_f32((uint32_t)stg[c][2]);
        const uint32_t w0 = (uint32_t)stg[c][0], w1 = (uint32_t)stg[c][1];
        *(i32x4_t*)(row + (((2 * p) ^ sw) << 3)) =
            i32x4_t{(int)fp4x2_to_bf16x2<0>(w0, sc), (int)fp4x2_to_bf16x2<1>(w0, sc),
                    (int)fp4x2_to_bf16x2<2>(w0, sc), (int)fp4x2_to_bf16x2<3>(w0, sc)};
        *(i32x4_t*)(row + (((2 * p + 1) ^ sw) << 3)) =
            i32x4_t{(int)fp4x2_to_bf16x2<0>(w1, sc), (int)fp4x2_to_bf16x2<1>(w1, sc),
                    (int)fp4x2_to_bf16x2<2>(w1, sc), (int)fp4x2_to_bf16x2<3>(w1, sc)};
      } else {
        uint32_t b[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) e4m3x4_to_bf16x4((uint32_t)stg[c][w], b[2 * w], b[2 * w + 1]);
        *(i32x4_t*)(row + (((2 * p) ^ sw) << 3)) = i32x4_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        *(i32x4_t*)(row + (((2 * p + 1) ^ sw) << 3)) = i32x4_t{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
      }
    }
  };
  // positives of tile t: quarter t & 3 of the 128-label bucket tile c0 / 128 + t / 4 (c0 is a
  // multiple of 128)
  auto yclear = [&](int buf) {
    if (tid < TJ) ybits[buf][tid] = 0u;
  };
  auto yscan = [&](int t, int buf) {
    const int64_t tb = c0 / TJ1 + (t >> 2);
    const uint32_t quarter = (uint32_t)(t & 3);
    const uint64_t e0 = tile_off[tb];
    const uint64_t e1 = tile_off[tb + 1] < (uint64_t)bucket_cap ? tile_off[tb + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 512) {
      const uint32_t v = bucket[e];
      const uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB && (jl >> 5) == quarter) atomicOr(&ybits[buf][jl & (TJ - 1)], 1u << b);
    }
  };

  float lsum = 0.0f;
  if (t0 < t1) {
    wload(t0);
    yclear(0); yclear(1); yclear(2); yclear(3);
    wstore(0);
    __syncthreads();
    yscan(t0, 0);
    __syncthreads();
  }
  // every prologue load done here (one wait), so that no wait for them lands inside the loop (the
  // compiler would otherwise wait on the vector-memory counter, which the loop's stores share,
  // every iteration)
  __builtin_amdgcn_s_waitcnt(0);
  for (int i = 0; t0 + i < t1; ++i) {
    const int t = t0 + i, buf = i & 1;
    const uint16_t* ws = Ws[buf];
    if (t + 1 < t1) wload(t + 1);

    // 1. the wave's partial logits over its K steps
    {
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int k = 0; k < NKW; ++k)
        acc = mfma_bf16(xf[k], *(const s16x8_t*)(ws + offF(NKW * wave + k)), acc);
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        Zs[wave][ig][lane] = f32x4_t{acc[4 * ig], acc[4 * ig + 1], acc[4 * ig + 2], acc[4 * ig + 3]};
    }
    __syncthreads();

    // 2. logits of accumulator registers 2 wave, 2 wave + 1 (summed in a fixed order), gradient
    {
      const int ig = wave >> 1, e0 = 2 * (wave & 1);
      float z0 = 0.0f, z1 = 0.0f;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const f32x4_t p = Zs[v][ig][lane];
        z0 += p[e0];
        z1 += p[e0 + 1];
      }
      const int b0 = 8 * ig + 4 * hi + e0;      // samples b0, b0 + 1 of label l32
      const bool jvalid = t * TJ + l32 < clen;
      const uint32_t yw = ybits[i & 3][l32];
      const bool y0 = (yw >> b0) & 1u, y1 = (yw >> (b0 + 1)) & 1u;
      const bool v0 = jvalid && b0 < B, v1 = jvalid && b0 + 1 < B;
      // the gradient forms chosen per wave as in the two-kernel forward: the short forms when every
      // element is valid and |z| <= 80 (<= 2: the small-argument form), else the exact selection
      float g0, g1;
      const float m = fmaxf(__builtin_fabsf(z0), __builtin_fabsf(z1));
      if (__builtin_amdgcn_ballot_w64(!(m <= 80.0f && v0 && v1)) == 0) {
        const uint32_t m0 = y0 ? 0x80000000u : 0u, m1 = y1 ? 0x80000000u : 0u;
        if (__builtin_amdgcn_ballot_w64(m > 2.0f) == 0) {
          g0 = bce_grad_small_m(z0, m0); g1 = bce_grad_small_m(z1, m1);
        } else {
          g0 = bce_grad_fast_m(z0, m0); g1 = bce_grad_fast_m(z1, m1);
        }
      } else {
        g0 = v0 ? bce_grad(z0, y0) : 0.0f;
        g1 = v1 ? bce_grad(z1, y1) : 0.0f;
      }
      if constexpr (LOSS) {
        if (v0) lsum += bce_loss(z0, y0);
        if (v1) lsum += bce_loss(z1, y1);
      }
      const uint32_t pk = pack_bf16x2(g0, g1);
      *(uint32_t*)(Gs + l32 * MB + ((((b0 >> 3) ^ gW) << 3) | (b0 & 7))) = pk;
      if (gout) {                              // diagnostic copy of the gradient codes, [B][gpitch]
        uint16_t* o = gout + (int64_t)b0 * gpitch + c0 + t * TJ + l32;
        if (v0) o[0] = (uint16_t)(pk & 0xffffu);
        if (v1) o[gpitch] = (uint16_t)(pk >> 16);
      }
    }
    __syncthreads();

    // 3. the tile's dX contribution over the wave's feature blocks
    {
      const s16x8_t gt0 = join(lds_read_tr16(Gs + offB0), lds_read_tr16(Gs + offB1));
      const s16x8_t gt1 = join(lds_read_tr16(Gs + offB0 + 16 * MB), lds_read_tr16(Gs + offB1 + 16 * MB));
#pragma unroll
      for (int f = 0; f < NFW; ++f) {
        const s16x8_t a0 = join(lds_read_tr16(ws + offA0[f]), lds_read_tr16(ws + offA1[f]));
        const s16x8_t a1 = join(lds_read_tr16(ws + offA0[f] + 16 * D), lds_read_tr16(ws + offA1[f] + 16 * D));
        accX[f] = mfma_bf16(a0, gt0, accX[f]);
        accX[f] = mfma_bf16(a1, gt1, accX[f]);
      }
    }
    // 4. the next tile (loaded at the top) into the other buffer, and its positives, before the
    // update (the staging registers are then free across it)
    if (t + 1 < t1) {
      wstore(buf ^ 1);
      yscan(t + 1, (i + 1) & 3);
    }
    // 5. per feature block, dW and the update of the wave's 32 x 32 block, in place (one block's dW
    // live at a time)
    {
      const s16x8_t g0 = *(const s16x8_t*)(Gs + offW[0]), g1 = *(const s16x8_t*)(Gs + offW[1]);
      const int ro = (t * TJ + l32) * RB;
#pragma unroll
      for (int f = 0; f < NFW; ++f) {
        f32x16_t accW = mfma_bf16(xT[f][0], g0, f32x16_t{});
        accW = mfma_bf16(xT[f][1], g1, accW);
        const int fb = NFW * wave + f, fU = 32 * fb;
        const int offUA[2] = {l32 * D + (((4 * fb) ^ swL) << 3) + 4 * hi, l32 * D + (((4 * fb + 2) ^ swL) << 3) + 4 * hi};
        const int offUB[2] = {l32 * D + (((4 * fb + 1) ^ swL) << 3) + 4 * hi,
                              l32 * D + (((4 * fb + 3) ^ swL) << 3) + 4 * hi};
        const uint64_t grp = ((uint64_t)(c0 + t * TJ + l32) * (uint64_t)D + (uint64_t)fU) >> 5;
        UpdState st;
        static_for<0, UPD_PHASES>([&](auto PH) {
          upd_phase<WF>(decltype(PH)::value, st, accW, ws, offUA, offUB, wres,
                        ro + (WF == W_MXFP4_ ? fU / 2 : fU * ESZ), ro + D / 2 + fU / 32, grp, hi, lr, seed, step);
        });
      }
    }

    yclear((i + 2) & 3);
    __syncthreads();
  }

  // the range's running dX partial back to its slot
#pragma unroll
  for (int i = 0; i < NFW; ++i)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig)
      *(f32x4_t*)(slot + ((NFW * wave + i) * 4 + ig) * 256) =
          f32x4_t{accX[i][4 * ig], accX[i][4 * ig + 1], accX[i][4 * ig + 2], accX[i][4 * ig + 3]};

  if constexpr (LOSS) {
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    if (tid == 0 && t0 < t1) {
      float s = 0.0f;
      for (int w = 0; w < 8; ++w) s += lred[w];
      loss_part[c0 / TJ + t0] = s;
    }
  }
}

#define LAUNCH_CHECK() do { if (hipGetLastError() != hipSuccess) return ELMO_EHIP_; } while (0)

template <int WF>
int run_single(const StepArgs& a, const StepLayout& s, uint8_t* ws, hipStream_t st) {
  uint8_t* W = (uint8_t*)a.W;
  const uint16_t* Xb = (const uint16_t*)(ws + s.xb);
  const uint8_t* Xq = WF == W_BF16_ ? (const uint8_t*)nullptr : ws + s.xq;
  const uint16_t* XbT = (const uint16_t*)(ws + s.xbt);
  const uint32_t* toff = (const uint32_t*)(ws + s.tile_off);
  const uint32_t* bucket = (const uint32_t*)(ws + s.bucket);
  float* part = (float*)(ws + s.part);
  float* lpart = (float*)(ws + s.loss);
  for (int64_t c0 = a.l0; c0 < a.l1; c0 += s.Cc) {
    const int clen = (int)((a.l1 - c0) < s.Cc ? (a.l1 - c0) : s.Cc);
    const int first = c0 == a.l0;
    kt_begin(KT_BWD, st, clen);
    auto launch = [&](auto NFW, auto LOSS) {
      hipLaunchKernelGGL((k_step_single<WF, decltype(NFW)::value, decltype(LOSS)::value>), dim3(s.NR1), dim3(512), 0,
                         st, W, c0, clen, Xb, Xq, XbT, toff, bucket, a.nnz, a.B, part, a.lr, a.seed, a.step, first,
                         lpart, a.Gout, a.L);
    };
    using N1 = std::integral_constant<int, 1>;
    using N2 = std::integral_constant<int, 2>;
    using N3 = std::integral_constant<int, 3>;
    if (a.loss) {
      if (a.D == 256) launch(N1{}, std::true_type{});
      else if (a.D == 512) launch(N2{}, std::true_type{});
      else launch(N3{}, std::true_type{});
    } else {
      if (a.D == 256) launch(N1{}, std::false_type{});
      else if (a.D == 512) launch(N2{}, std::false_type{});
      else launch(N3{}, std::false_type{});
    }
    LAUNCH_CHECK();
    kt_end(KT_BWD, st);
  }
  return ELMO_OK_;
}

template int run_single<W_BF16_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
template int run_single<W_E4M3_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
template int run_single<W_MXFP4_>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);

}  // namespace elmo
