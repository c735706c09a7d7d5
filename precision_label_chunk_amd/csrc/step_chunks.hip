// The two chunk kernels of the chunked, fused XMC classifier-head training step on gfx950, and the
// chunk scheduler that launches them. The file is compiled once per (padded batch, weight format)
// pair: the build defines ELMO_MB and ELMO_WF, and each object holds that pair's instantiation of
// run_chunks (the variants then compile in parallel).
//
// Method: "ELMO: Efficiency via Low-precision and Peak Memory Optimization in Large Output Spaces"
// (summary page, "Approach": pure BF16/FP8 classifier with stochastic rounding, no momentum, the
// classifier gradient fused with the SGD update, the label dimension chunked to cut transient
// memory; arXiv abstract: "gradient fusion and chunking").
//
// Per label chunk [c0, c0 + clen) two kernels run on the caller's stream:
//   k_fwd_g       label tiles of 128 x all B: Z = X~ W_c^T on the matrix cores (BF16, or E4M3 in
//                 FP8 mode), then G = BF16(sigmoid(Z) - Y) in the epilogue straight from the
//                 accumulators; writes the chunk's G (the only chunk-sized transient).
//   k_bwd_update  (d-slice, label range) work-groups: one LDS-staged G tile feeds both backward
//                 contractions — dX^T += W_old^T G^T (FP32 accumulators that live across the whole
//                 label range) and dW^T = X^T G — and dW goes straight into t = fmaf(-lr, dW, w)
//                 and the stochastic rounding; the updated weights are written back in place with
//                 coalesced 16-byte stores. dW is never stored outside the work-group.
// Label handling, X preparation and the final dX reduction are small kernels around them
// (step_kernels.hip).
#include "step_kernels.hpp"

#include <type_traits>

#include "fwd_mx.hpp"
#include "fwd_tile.hpp"
#include "mfma.hpp"
#include "numerics.hpp"
#include "update.hpp"

namespace elmo {

// ------------------------------------------------------------------------------------------------
// forward + gradient: Z = X~ W_c^T, G = BF16(sigmoid(Z) - Y)
// ------------------------------------------------------------------------------------------------
// Gradient of one 32 x 32 accumulator block: lane (l32, hi) holds label l32 of the block and
// samples bb + 8 (i/4) + 4 hi + i%4 in register i; yw holds the positives of samples bb .. bb+31 of
// that label. Padding (samples >= B, labels past the chunk) gets 0. The exact form is needed only
// for |z| > 80: one wave-uniform test per block (every |z| <= 80, every sample and label valid)
// keeps the common case free of branches and selects, and a second one takes the shorter
// small-argument form when every |z| of the block is at most 2.
__device__ __forceinline__ void fwd_grad_block(const f32x16_t& a, uint32_t yw, bool jvalid, int bb, int B, int hi,
                                               float (&gv)[16]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, __builtin_fabsf(a[i]));
  const bool common = m <= 80.0f && jvalid && bb + 32 <= B;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!common) == 0, 1)) {
    // every element in range and valid: no select; label bit bl of yw moved to bit 31
    const uint32_t yh = yw >> (4 * hi);
    if (__builtin_amdgcn_ballot_w64(yh != 0u) == 0) {
      // (the usual block: no positives, so no label bits and no sign operations)
      if (__builtin_amdgcn_ballot_w64(m > 2.0f) == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) gv[i] = bce_grad_small_y0(a[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) gv[i] = bce_grad_fast_y0(a[i]);
      }
    } else if (__builtin_amdgcn_ballot_w64(m > 2.0f) == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) gv[i] = bce_grad_small_m(a[i], yh << (31 - (8 * (i >> 2) + (i & 3))));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) gv[i] = bce_grad_fast_m(a[i], yh << (31 - (8 * (i >> 2) + (i & 3))));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int bl = 8 * (i >> 2) + 4 * hi + (i & 3);
      gv[i] = jvalid && (bb + bl < B) ? bce_grad(a[i], (yw >> bl) & 1u) : 0.0f;
    }
  }
}

// The chunk gradient buffer G holds, per 64-label backward tile, MB x 64 BF16 values in blocks of
// 32 labels x 32 samples, each the 2 KiB that one wave's accumulator block packs to:
//   tile T = label >> 6, block (jb = (label >> 5) & 1, sb = sample >> 5) at elements
//   T 64 MB + (jb MB / 32 + sb) 1024; within it, half u at 512 u, lane (l, h) at 8 lane: label
//   32 (label >> 5) + l, samples 32 sb + 16 u + 8 h .. + 7.
// Packing pairs to BF16 and swapping register groups 1 <-> 0 and 3 <-> 2 across the lane halves
// leaves each lane exactly those 8 samples of its label for u = 0 and 1, so each half of a block
// leaves in one 16-byte store per lane, 1 KiB contiguous per wave. jc is any label of the block
// (chunk-relative), bb its first sample.
__device__ __forceinline__ void fwd_store_block(const float (&gv)[16], uint16_t* G, int MB, int jc, int bb, int lane) {
  uint32_t pk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(gv[2 * k], gv[2 * k + 1]);
  uint16_t* blk = G + (int64_t)(jc >> 6) * 64 * MB + (((jc >> 5) & 1) * (MB / 32) + (bb >> 5)) * 1024 + lane * 8;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * u], pk[4 * u + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * u + 1], pk[4 * u + 3], false, false);
    const i32x4_t out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    *(i32x4_t*)(blk + 512 * u) = out;
  }
}

// The epilogue of a 128-label forward tile (4 waves; wave (wb, wj) holds samples wb RW .. + RW - 1
// and labels wj CW .. + CW - 1 of the tile in 32 x 32 accumulator blocks): the gradient straight
// from the accumulators, block by block, into the chunk buffer G. The loss partial of the tile
// goes to loss_part[lslot].
template <int MB, int RW, int CW, bool LOSS, bool ZOUT>
__device__ __forceinline__ void fwd_epilogue(f32x16_t (&acc)[RW / 32][CW / 32], uint8_t* smem,
                                             const uint32_t* ybits, float* lred, int tid, int wb, int wj,
                                             int jbase, int clen, int B, int64_t c0, uint16_t* __restrict__ G,
                                             int64_t gpitch, float* __restrict__ loss_part, int64_t lslot,
                                             float* __restrict__ Z, uint16_t* __restrict__ Gout, int64_t zpitch,
                                             int64_t zoff) {
  constexpr int MI = RW / 32, NI = CW / 32;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  (void)smem; (void)gpitch;
  float lsum = 0.0f;
  // (unrolled at compile time: with the loss inlined, a pragma-directed unroll of 4 x 2 blocks at
  // 256 samples exceeds the compiler's size limit, and the accumulators would then be indexed at
  // run time, that is, through scratch memory)
  static_for<0, MI>([&](auto MIc) {
    constexpr int mi = decltype(MIc)::value;
    static_for<0, NI>([&](auto NIc) {
      constexpr int ni = decltype(NIc)::value;
      const int jl = wj * CW + ni * 32 + l32;
      const bool jvalid = jbase + jl < clen;
      const int bb = wb * RW + mi * 32;
      const uint32_t yw = ybits[jl * (MB / 32) + (bb >> 5)];
      float gv[16];
      fwd_grad_block(acc[mi][ni], yw, jvalid, bb, B, hi, gv);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int bl = 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool valid = jvalid && (bb + bl < B);
        const bool y = (yw >> bl) & 1u;
        const float z = acc[mi][ni][i];
        if constexpr (LOSS) if (valid) lsum += bce_loss(z, y);
        if constexpr (ZOUT) {
          const int64_t lab = c0 + jbase + jl;
          if (valid && lab >= zoff) {
            const int64_t o = (int64_t)(bb + bl) * zpitch + (lab - zoff);
            if (Z) Z[o] = z;
            if (Gout) Gout[o] = (uint16_t)f32_to_bf16_rne(gv[i]);
          }
        }
      }
      if constexpr (!ZOUT) fwd_store_block(gv, G, MB, jbase + jl, bb, lane);
    });
  });
  if constexpr (LOSS) {
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    if (tid == 0) loss_part[lslot] = ((lred[0] + lred[1]) + lred[2]) + lred[3];
  }
}

template <int MB, int WF, bool LOSS, bool ZOUT>
__global__ __launch_bounds__(256, 2) void k_fwd_g(const uint8_t* __restrict__ W, const uint8_t* __restrict__ Xf,
                                               int D, int64_t c0, int clen,
                                               const uint32_t* __restrict__ tile_off,
                                               const uint32_t* __restrict__ bucket, int64_t bucket_cap,
                                               int B, uint16_t* __restrict__ G, int64_t gpitch,
                                               float* __restrict__ loss_part,
                                               float* __restrict__ Z, uint16_t* __restrict__ Gout,
                                               int64_t zpitch, int64_t zoff) {
  constexpr int WB = MB >= 64 ? 2 : 1, WJ = 4 / WB;
  constexpr int RW = MB / WB, CW = TJ1 / WJ;   // wave tile: RW samples x CW labels
  constexpr int MI = RW / 32, NI = CW / 32;
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
  // K slice: small enough for two work-groups per CU; 128 bytes (64 BF16 elements, half the
  // barriers) where the LDS stages of 256 rows still leave room for the second work-group
  constexpr int KS = (MB <= 128 && WF == W_BF16_) ? 128 : 64;
  __shared__ __attribute__((aligned(16))) uint8_t smem[fwd_smem_bytes(MB, KS)];
  __shared__ uint32_t ybits[TJ1 * (MB / 32)];    // positives, label-major: bit b & 31 of word [j][b >> 5]
  __shared__ float lred[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wb = wave / WJ, wj = wave % WJ;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = blockIdx.x;
  const int64_t tg = c0 / TJ1 + tile;          // global 128-label tile index
  const int jbase = tile * TJ1;                // first label of the tile, relative to c0
  const int64_t rowbytes = (int64_t)D * ESZ;

  f32x16_t acc[MI][NI];
  // the tile's positives into ybits while the first K slices load
  auto scan = [&]() {
    for (int i = tid; i < TJ1 * (MB / 32); i += 256) ybits[i] = 0u;
    __syncthreads();
    const uint64_t e0 = tile_off[tg];
    const uint64_t e1 = tile_off[tg + 1] < (uint64_t)bucket_cap ? tile_off[tg + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 256) {
      uint32_t v = bucket[e];
      uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB) atomicOr(&ybits[jl * (MB / 32) + (b >> 5)], 1u << (b & 31));
    }
  };
  fwd_tile<MB, WF, RW, CW, KS>(acc, smem, W + (c0 + jbase) * rowbytes, clen - jbase, Xf, rowbytes, tid, wb, wj, scan);

  fwd_epilogue<MB, RW, CW, LOSS, ZOUT>(acc, smem, ybits, lred, tid, wb, wj, jbase, clen, B, c0, G, gpitch, loss_part, tg,
                                      Z, Gout, zpitch, zoff);
}

// ------------------------------------------------------------------------------------------------
// forward + gradient for MX-scaled FP4 weights (E2M1 elements, one E8M0 scale per 32 features)
// ------------------------------------------------------------------------------------------------
// One work-group per 128-label tile, 4 waves (the wave tiles of k_fwd_g), the logits on the scaled
// matrix cores (mx_logit_tile: every lane loads its own operand fragments, the features from the
// E4M3 copy in the workspace, which stays in L2, the weight rows once per work-group); rows past
// the chunk read as zero. The epilogue is the tiled forward's.
template <int MB, bool LOSS, bool ZOUT>
__global__ __launch_bounds__(256, 2) void k_fwd_mx(const uint8_t* __restrict__ W, const uint8_t* __restrict__ Xq,
                                                int D, int64_t c0, int clen,
                                                const uint32_t* __restrict__ tile_off,
                                                const uint32_t* __restrict__ bucket, int64_t bucket_cap,
                                                int B, uint16_t* __restrict__ G, int64_t gpitch,
                                                float* __restrict__ loss_part,
                                                float* __restrict__ Z, uint16_t* __restrict__ Gout,
                                                int64_t zpitch, int64_t zoff) {
  constexpr int WB = MB >= 64 ? 2 : 1, WJ = 4 / WB;
  constexpr int RW = MB / WB, CW = TJ1 / WJ;   // wave tile: RW samples x CW labels
  constexpr int MI = RW / 32, NI = CW / 32;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * 64 * 144];   // the epilogue's G staging
  __shared__ uint32_t ybits[TJ1 * (MB / 32)];
  __shared__ float lred[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wb = wave / WJ, wj = wave % WJ;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = blockIdx.x;
  const int64_t tg = c0 / TJ1 + tile;
  const int jbase = tile * TJ1;
  const int rb = D / 2 + D / 32;                     // bytes per weight row
  const int nvalid = clen - jbase < TJ1 ? clen - jbase : TJ1;
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + (c0 + jbase) * (int64_t)rb, nvalid * rb);
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(Xq, MB * D);

  for (int i = tid; i < TJ1 * (MB / 32); i += 256) ybits[i] = 0u;
  __syncthreads();
  {
    const uint64_t e0 = tile_off[tg];
    const uint64_t e1 = tile_off[tg + 1] < (uint64_t)bucket_cap ? tile_off[tg + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 256) {
      const uint32_t v = bucket[e];
      const uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB) atomicOr(&ybits[jl * (MB / 32) + (b >> 5)], 1u << (b & 31));
    }
  }

  f32x16_t acc[MI][NI];
  mx_logit_tile<MI, NI>(acc, xres, wb * RW, D, wres, wj * CW, rb, l32, hi);
  __syncthreads();                                   // label bits complete
  fwd_epilogue<MB, RW, CW, LOSS, ZOUT>(acc, smem, ybits, lred, tid, wb, wj, jbase, clen, B, c0, G, gpitch, loss_part, tg,
                                      Z, Gout, zpitch, zoff);
}

// ------------------------------------------------------------------------------------------------
// forward + gradient with the features stationary in registers (E4M3 or MXFP4 weights, 256
// samples, D = 768)
// ------------------------------------------------------------------------------------------------
// The tiled forward above reloads every feature row for every 128-label tile and waits on those
// loads in each K slice. Here each work-group holds all 256 E4M3 feature rows in registers for the
// whole launch (wave w: samples 32 w .. 32 w + 31, lane (l32, hi) the MFMA A fragments of row
// 32 w + l32, 32 bytes per 64-byte K step: D / 8 registers) and streams the chunk's weights through
// LDS in 64-label tiles, two tile buffers: tile t's rows are loaded (into registers) at the start
// of iteration t - 1 and written to LDS at its end, into the buffer tile t - 1 used. One
// work-group per CU takes tiles blockIdx.x, + gridDim.x, ...
// The waves come in two groups of four, one wave of each per SIMD, in complementary phases: in
// iteration i group A (waves 0-3) runs tile i's MFMAs and then its gradient epilogue, group B (4-7)
// runs the epilogue of tile i - 1 and then tile i's MFMAs, so that on every SIMD one wave's matrix
// work overlaps the other's epilogue arithmetic. One barrier per iteration. The positives of tile
// i + 1 are gathered into label bits during iteration i (four buffers: A reads tile i's, B tile
// i - 1's, i + 1's is being filled and i + 2's cleared).
// MXFP4 weights: a tile's 64 rows (17 D / 32 bytes each) are contiguous in memory and 16-byte
// aligned, so they are loaded as one flat run of 16-byte chunks and written to LDS in 8-byte halves
// (which never straddle a row) at a row pitch of 432 bytes (108 banks: 16 consecutive rows' 16-byte
// fragment reads fall on distinct banks). Per MFMA a lane reads its 16 code bytes; the 24 scale
// bytes of its row are read once per tile and permuted so that dword m holds the lane's scales of
// K steps 4m .. 4m + 3, each selected by the instruction's byte select. The features take the E4M3
// operand's K order beside an FP4 operand.
constexpr int XS_TJ = 64;                                      // labels per tile

// NK: 64-byte K steps of the FP8 MFMA (D = 64 NK; the features take 8 NK registers)
template <int WF, int NK, bool LOSS, bool ZOUT>
__global__ __launch_bounds__(512, 1) void k_fwd_xs(const uint8_t* __restrict__ W, const uint8_t* __restrict__ Xq,
                                                int D, int64_t c0, int clen,
                                                const uint32_t* __restrict__ tile_off,
                                                const uint32_t* __restrict__ bucket, int64_t bucket_cap,
                                                int B, uint16_t* __restrict__ G, int64_t gpitch,
                                                float* __restrict__ loss_part,
                                                float* __restrict__ Z, uint16_t* __restrict__ Gout,
                                                int64_t zpitch, int64_t zoff) {
  constexpr int MB = 256;
  constexpr bool MX = WF == W_MXFP4_;
  constexpr int D_ = 64 * NK;
  constexpr int RB = MX ? D_ / 2 + D_ / 32 : D_;     // bytes per weight row
  static_assert(!MX || (XS_TJ * RB) % 16 == 0, "MXFP4 tiles are whole 16-byte chunks");
  // LDS row pitch: 16 consecutive rows on distinct banks for the 16-byte fragment reads
  constexpr int PITCH = MX ? 432 : D_ + 16;
  static_assert(PITCH >= RB && (PITCH / 4) % 8 == 4, "pitch: whole rows, an odd number of 4-bank groups");
  constexpr int PPR = D_ / 16;                        // (E4M3) 16-byte parts per weight row
  constexpr int NCH = MX ? XS_TJ * RB / 16 : XS_TJ * PPR;   // 16-byte chunks per tile
  constexpr int CPT = (NCH + 511) / 512;              // 16-byte weight chunks per thread and tile
  __shared__ __attribute__((aligned(16))) uint8_t Ws[2][XS_TJ * PITCH];
  __shared__ uint32_t ybits[4][XS_TJ * (MB / 32)];   // label-major: bit b & 31 of word [j][b >> 5]
  __shared__ float lred[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                          // 0: MFMAs then epilogue; 1: epilogue then MFMAs
  const int l32 = lane & 31, hi = lane >> 5;
  const int bb = 32 * wave;                           // the wave's first sample
  const int ntl = (clen + XS_TJ - 1) / XS_TJ;         // tiles of the chunk
  const int nmy = ntl > (int)blockIdx.x ? (ntl - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  auto tile_of = [&](int i) { return (int)blockIdx.x + i * (int)gridDim.x; };
  (void)D;
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + c0 * (int64_t)RB, clen * RB);
  constexpr int OOB = 0x7ffffff0;

  // weight tile staging through registers: chunk c of this thread is ci = tid + 512 c, row ci / PPR,
  // part ci % PPR (E4M3), or bytes 16 ci .. 16 ci + 15 of the tile's flat rows (MXFP4); rows past
  // the chunk read as zero (resource bound), chunks past the tile are idle
  i32x4_t stg[CPT];
  auto wload = [&](int t, i32x4_t (&stg)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + 512 * c;
      if constexpr (MX) {
        stg[c] = buffer_load16(wres, ci < NCH ? t * XS_TJ * RB + ci * 16 : OOB);
      } else {
        const int row = ci / PPR, part = ci % PPR;
        stg[c] = buffer_load16(wres, row < XS_TJ ? (t * XS_TJ + row) * D_ + part * 16 : OOB);
      }
    }
  };
  auto wstore = [&](int buf, const i32x4_t (&stg)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + 512 * c;
      if constexpr (MX) {
        if (ci < NCH) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int b = ci * 16 + 8 * h, row = b / RB, off = b - row * RB;
            *(i32x2_t*)(&Ws[buf][row * PITCH + off]) = i32x2_t{stg[c][2 * h], stg[c][2 * h + 1]};
          }
        }
      } else {
        const int row = ci / PPR, part = ci % PPR;
        if (row < XS_TJ) *(i32x4_t*)(&Ws[buf][row * PITCH + part * 16]) = stg[c];
      }
    }
  };
  // positives of tile t (64 labels: half (c0 / 64 + t) & 1 of 128-label bucket tile (c0 / 64 + t) >> 1)
  auto yclear = [&](int buf) {
    for (int i = tid; i < XS_TJ * (MB / 32); i += 512) ybits[buf][i] = 0u;
  };
  auto yscan = [&](int t, int buf) {
    const int64_t g64 = c0 / XS_TJ + t;
    const int64_t tb = g64 >> 1;
    const uint32_t half = (uint32_t)(g64 & 1);
    const uint64_t e0 = tile_off[tb];
    const uint64_t e1 = tile_off[tb + 1] < (uint64_t)bucket_cap ? tile_off[tb + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 512) {
      const uint32_t v = bucket[e];
      const uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB && (jl >> 6) == half)
        atomicOr(&ybits[buf][(jl & (XS_TJ - 1)) * (MB / 32) + (b >> 5)], 1u << (b & 31));
    }
  };

  // prologue: tile 0, then the stationary feature fragments, all in flight together (a tile this
  // work-group does not have lies past the chunk and reads as zero); the tile's LDS writes wait
  // only for the tile loads, which were issued first, so the feature loads complete under the LDS
  // writes, the barriers and the first MFMAs, each MFMA waiting only for its own fragment
  i32x8_t xf[NK];
  wload(tile_of(0), stg);
  {
    // E4M3 beside E4M3: bytes 32 hi .. +31 of each K step; beside FP4: 16 hi .. +15 and 32 + 16 hi .. +15,
    // as the step's preparation lays them out: part p of K step kk at ((wave NK + kk) 2 + p) KiB
    // (one lane offset, the K step's in the instructions' scalar offsets)
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(Xq, MB * D_);
    const int xo = (wave * NK * 2 * 64 + lane) * 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const i32x4_t a0 = buffer_load16(xres, xo, 2 * kk * 1024), a1 = buffer_load16(xres, xo, (2 * kk + 1) * 1024);
      xf[kk] = i32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  }
  yclear(0); yclear(1); yclear(2);
  wstore(0, stg);
  __syncthreads();
  if (nmy > 0) yscan(tile_of(0), 0);
  __syncthreads();

  f32x16_t acc[2];
  float lsum = 0.0f;
  // the tile's 2 NK MFMAs (slot z: K step z / 2, label block z % 2), each slot's weight fragment read
  // from LDS two slots ahead; a scheduling fence closes every slot so that the reads stay spread
  auto mfmas_mx = [&](int buf) {
    acc[0] = f32x16_t{}; acc[1] = f32x16_t{};
    const uint8_t* wb = &Ws[buf][l32 * PITCH + hi * 16];
    // scale dword m of label block ni: bytes 2 (4m + j) + hi of the row's scales, j = 0..3
    uint32_t scl[2][NK / 4];
    static_assert(NK % 4 == 0, "whole scale dwords");
    const uint32_t psel = hi ? 0x07050301u : 0x06040200u;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const uint8_t* sp = wb - hi * 16 + ni * 32 * PITCH + D_ / 2;
#pragma unroll
      for (int m = 0; m < NK / 4; ++m) {
        const i32x2_t r = *(const i32x2_t*)(sp + 8 * m);
        scl[ni][m] = __builtin_amdgcn_perm((uint32_t)r[1], (uint32_t)r[0], psel);
      }
    }
    auto rd = [&](int z) { return *(const i32x4_t*)(wb + (z & 1) * 32 * PITCH + (z >> 1) * 32); };
    constexpr int NS = 2 * NK;
    i32x4_t f[3];
    f[0] = rd(0); f[1] = rd(1);
    static_for<0, NS>([&](auto Z) {
      constexpr int z = decltype(Z)::value, kk = z >> 1;
      if constexpr (z + 2 < NS) f[(z + 2) % 3] = rd(z + 2);
      acc[z & 1] = mfma_e4m3_fp4_sel<kk % 4>(xf[kk], f[z % 3], acc[z & 1], (int)scl[z & 1][kk / 4]);
      sched_fence();
    });
  };
  auto mfmas = [&](int buf) {
    if constexpr (MX) {
      mfmas_mx(buf);
      return;
    }
    acc[0] = f32x16_t{}; acc[1] = f32x16_t{};
    const uint8_t* wb = &Ws[buf][l32 * PITCH + hi * 32];
    auto rd = [&](int z) {
      const uint8_t* p = wb + (z & 1) * 32 * PITCH + (z >> 1) * 64;
      const i32x4_t b0 = *(const i32x4_t*)p, b1 = *(const i32x4_t*)(p + 16);
      return i32x8_t{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    };
    constexpr int NS = 2 * NK;
    i32x8_t f[3];
    f[0] = rd(0); f[1] = rd(1);
    static_for<0, NS>([&](auto Z) {
      constexpr int z = decltype(Z)::value;
      if constexpr (z + 2 < NS) f[(z + 2) % 3] = rd(z + 2);
      acc[z & 1] = mfma_e4m3(xf[z >> 1], f[z % 3], acc[z & 1]);
      sched_fence();
    });
  };
  auto epilogue = [&](int t, int buf) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int jl = ni * 32 + l32;
      const int jc = t * XS_TJ + jl;                  // label within the chunk
      const bool jvalid = jc < clen;
      const uint32_t yw = ybits[buf][jl * (MB / 32) + wave];
      float gv[16];
      fwd_grad_block(acc[ni], yw, jvalid, bb, B, hi, gv);
      if constexpr (LOSS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int bl = 8 * (i >> 2) + 4 * hi + (i & 3);
          if (jvalid && (bb + bl < B)) lsum += bce_loss(acc[ni][i], (yw >> bl) & 1u);
        }
      }
      if constexpr (ZOUT) {
        // (diagnostic) element (sample bb + bl, label c0 + jc) at row-major [B][zpitch] offset
        // (bb + bl) zpitch + c0 + jc - zoff, from one base per lane and row steps of zpitch
        const int64_t lab = c0 + jc;
        const bool lok = jvalid && lab >= zoff;
        const int64_t base = (int64_t)(bb + 4 * hi) * zpitch + (lab - zoff);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + (i & 3);
          if (lok && bb + 4 * hi + r < B) {
            const int64_t o = base + r * zpitch;
            if (Z) Z[o] = acc[ni][i];
            if (Gout) Gout[o] = (uint16_t)f32_to_bf16_rne(gv[i]);
          }
        }
      }
      if constexpr (!ZOUT) fwd_store_block(gv, G, MB, jc, bb, lane);
    }
  };

  // (the diagnostic variant, whose stores take more registers, writes the weight tile to LDS right
  // after loading it: the same arithmetic, without the loads in flight across the iteration)
  constexpr bool LATE_STORE = !ZOUT;
  for (int i = 0; i <= nmy; ++i) {
    if (i + 1 < nmy) {
      wload(tile_of(i + 1), stg);
      if constexpr (!LATE_STORE) wstore((i + 1) & 1, stg);
    }
    // group A: MFMAs of tile i, then its epilogue; group B: epilogue of tile i - 1, then MFMAs of tile i
    const int ie = i - grp;                           // the tile index whose epilogue this wave runs
    if (grp == 0 && i < nmy) mfmas(i & 1);
    if (ie >= 0 && ie < nmy) epilogue(tile_of(ie), ie & 3);
    if (grp == 1 && i < nmy) mfmas(i & 1);
    if constexpr (LATE_STORE) if (i + 1 < nmy) wstore((i + 1) & 1, stg);
    if (i + 1 < nmy) yscan(tile_of(i + 1), (i + 1) & 3);
    yclear((i + 2) & 3);
    __syncthreads();
  }

  if constexpr (LOSS) {
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int w = 0; w < 8; ++w) s += lred[w];
      loss_part[c0 / XS_TJ + blockIdx.x] = s;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// backward + fused update over one d-slice and one label range of the chunk
// ------------------------------------------------------------------------------------------------
// Work-group: NH * DS/32 waves. The NH waves of feature block fb own the 32 features
// [dsl + 32 fb, +32) of the slice and share the two backward contractions of every tile; with
// NH = 2 (two waves per SIMD for DS = 128, so that one wave's update arithmetic fills the other's
// MFMA and LDS waits) wave half h computes dW of label block h over all samples and dX of sample
// half h over all the tile's labels:
//   dW^T[d][j]  = sum_b X^T[d][b] G[b][j]      2/NH 32-label blocks, K = MB samples  (MB/8/NH MFMAs)
//   dX^T[d][b] += sum_j W^T[d][j] G^T[j][b]    MB/32/NH sample blocks, K = 64 labels (MB/8/NH MFMAs)
// with A = stationary X^T fragments in registers (dW), B = G rows by ds_read_b128 (dW), and
// A = W^T, B = G^T by ds_read_b64_tr_b16 (dX). Per 64-label tile t:
//   G tile  the chunk buffer's 64-label tile (contiguous, in the forward's 32 x 32 blocks), in LDS
//           as [64][MB] BF16 label-major rows, double buffered in two
//           LDS arrays used alternately by an unrolled pair of tiles; staged through registers
//           (loaded at the start of the previous tile, written at its end) rather than with
//           global_load_lds, whose in-flight LDS writes make the compiler drain every LDS read
//           before each MFMA;
//   W tile  [64][DS] decoded to BF16 in LDS, three buffers: tile t's stays intact through tile t+1,
//           whose MFMAs its update overlaps, while tile t+2's is being staged.
// The tile's MFMAs run in slots (dW and dX alternating), each slot's LDS operands read PFS slots
// ahead, and the update of the wave's label blocks of the previous tile (UPD_PHASES phases of VALU
// work per block: RNG, rounding, stores) spread over the slots; a scheduling fence closes every
// slot so that the compiler keeps this interleaving. dW never leaves the registers; one barrier
// per tile.
template <int MB, int WF, int DS, int NH>
__global__ __launch_bounds__(DS * 2 * NH) void k_bwd_update(uint8_t* __restrict__ W, int D, int64_t c0, int clen,
                                                            const uint16_t* __restrict__ XbT,
                                                            const uint16_t* __restrict__ G,
                                                            float* __restrict__ part, int NR, int NS, float lr,
                                                            uint64_t seed, uint64_t step, int first) {
  constexpr int NFB = DS / 32;                 // feature blocks
  constexpr int NW = NFB * NH, NT = 64 * NW;   // waves, threads
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;   // (MXFP4: the staging and stores below have their own forms)
  constexpr int NB = MB / 32;                  // sample blocks
  constexpr int NJB = 2 / NH;                  // label blocks per wave (dW, update)
  constexpr int NBW = NB / NH;                 // sample blocks per wave (dX)
  constexpr int KK = MB / 16;                  // dW K steps per label block
  constexpr int NDW = NJB * KK;                // dW MFMAs per tile
  constexpr int KXN = TJ2 / 16;                // dX K steps
  constexpr int NDX = KXN * NBW;               // dX MFMAs per tile
  static_assert(NH == 1 || NH == 2, "one or two waves per feature block");
  static_assert(NBW >= 1 && NDW == NDX, "slots alternate dW and dX");
  constexpr int NSLOT = NDW + NDX;
  constexpr int PFS = NH == 2 ? 2 : 4;         // operand prefetch distance (slots)
  constexpr int GTE = TJ2 * MB;                // G tile elements
  constexpr int GCPR = MB / 8;                 // 16-byte chunks per G row
  constexpr int GPT = TJ2 * GCPR / NT;         // G chunks per thread
  // global W items per tile row: 16-byte chunks (BF16, E4M3), 16-element parts (MXFP4: 8 code bytes)
  constexpr int WCPR = WF == W_MXFP4_ ? DS / 16 : DS * ESZ / 16;
  constexpr int WPT = TJ2 * WCPR / NT;         // W chunks per thread
  constexpr int NOW = KK < 8 ? KK : 8;         // distinct dW operand offsets per lane
  constexpr int NOB = NBW < 4 ? NBW : 4;       // distinct dX operand offsets per lane and row
  static_assert(GPT >= 1 && WPT >= 1 && TJ2 == 64, "tile split");
  __shared__ __attribute__((aligned(1024))) uint16_t Gs0[GTE];
  __shared__ __attribute__((aligned(1024))) uint16_t Gs1[GTE];
  __shared__ __attribute__((aligned(1024))) uint16_t Ws[3][TJ2 * DS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dblk = wave % NFB, h = wave / NFB;  // feature block, wave half
  const int l32 = lane & 31, hi = lane >> 5, q = lane >> 4, li = lane & 15;
  // work-groups of one label range share its G tiles: dispatch is round-robin over the 8 XCDs, so
  // number the (range, slice) pairs XCD-major, consecutive on each XCD; at most one range per XCD
  // boundary is split between two L2s
  const int g = blockIdx.x, xcd = g & 7, kq = g >> 3;
  const int lin = xcd * (int)(gridDim.x >> 3) + kq;
  const int r = lin / NS, s = lin % NS;
  if (r >= NR) return;
  const int nt = (clen + TJ2 - 1) / TJ2;
  const int t0 = (int)((int64_t)nt * r / NR), t1 = (int)((int64_t)nt * (r + 1) / NR);
  const int dsl = s * DS;
  const int rowbytes = (int)w_row_bytes(WF, D);
  // the chunk's weight rows: rows past the chunk's end (the ragged last tile) load as zero and
  // drop their stores
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + c0 * (int64_t)rowbytes, clen * rowbytes);
  const int jb0 = NH == 2 ? h : 0;             // first label block of this wave
  const int nb0 = h * NBW;                     // first sample block of this wave

  // stationary X^T fragments of this wave's 32 features: lane (d, 8 samples), from the step
  // preparation's fragment-ordered copy (sample step kk of feature block fb at (fb MB / 16 + kk) KiB)
  s16x8_t xT[KK];
  {
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(XbT, MB * D * 2);
    const int xo = (((dsl + dblk * 32) >> 5) * (MB / 16) * 64 + lane) * 16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) xT[kk] = __builtin_bit_cast(s16x8_t, buffer_load16(xres, xo, kk * 1024));
  }
  // dX^T accumulators, starting from this range's running partial sum (a fixed slot per range:
  // deterministic; zero in the step's first chunk, where every slot has a range), read after the
  // first tile's staging loads have been issued (so that the tile's LDS writes and first dW MFMAs
  // do not wait for the 128 KiB of partials: the vector-memory counter retires in order) and
  // stored back at the end. The partial keeps the accumulators' own
  // layout, lane l's registers 4 ig .. 4 ig + 3 of sample block sb at ((sb * 4 + ig) * 64 + l) * 4
  // within the wave's feature block, so that every access is 1 KiB contiguous.
  // With four sample blocks per wave and an even number of feature blocks, each wave takes a 2 x 2
  // square of (feature block, sample block) pairs instead of one feature block's four sample
  // blocks, so that every A (W^T) and B (G^T) fragment feeds two MFMAs: 4 fragment reads per 4
  // MFMAs instead of 5. Accumulator a holds feature block xfb(a) of the slice, sample block xsb(a).
  constexpr bool SQ = NH == 2 && NBW == 4 && NFB % 2 == 0;
  const int fp = SQ ? wave % (NFB / 2) : 0, sp = SQ ? wave / (NFB / 2) : 0;
  auto xfb = [&](int a) { return SQ ? 2 * fp + (a >> 1) : dblk; };
  auto xsb = [&](int a) { return SQ ? 2 * sp + (a & 1) : nb0 + a; };
  float* slot = part + (int64_t)r * (D / 32) * (MB * 32) + 4 * lane;
  auto pslot = [&](int a, int ig) { return slot + (dsl / 32 + xfb(a)) * (MB * 32) + (xsb(a) * 4 + ig) * 256; };
  f32x16_t accX[NBW];
  // (through a resource of zero bytes in the first chunk, which reads zeros without a branch per load)
  const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(part + (int64_t)r * (D / 32) * (MB * 32), first ? 0 : D * MB * 4);
  auto init_acc = [&]() {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int off = ((dsl / 32 + xfb(nb)) * (MB * 32) + (xsb(nb) * 4 + ig) * 256 + 4 * lane) * 4;
        const f32x4_t o = __builtin_bit_cast(f32x4_t, buffer_load16(pres, off));
        accX[nb][4 * ig] = o[0]; accX[nb][4 * ig + 1] = o[1]; accX[nb][4 * ig + 2] = o[2]; accX[nb][4 * ig + 3] = o[3];
      }
  };

  // loop-invariant LDS element offsets (rows of both label blocks share the swizzle: it only
  // depends on the row's low 4 bits)
  //   dW operand B: G row jb*32 + l32, chunk 2 kk + hi  ->  16 (kk ^ gW1) + 8 (hi ^ gW0)
  const int gW = row_swz<MB / 8>(l32);
  int offW[NOW];
#pragma unroll
  for (int k = 0; k < NOW; ++k) offW[k] = (jb0 * 32 + l32) * MB + 8 * (hi ^ (gW & 1)) + 16 * (k ^ (gW >> 1));
  //   dX operands (transposing reads): rows jX and jX + 4 of each 16-label K step
  const int jX = 8 * (q >> 1) + (li >> 2);
  //     A = W^T: features 32 fb + 16 (q&1) + 4 (li&3) .. +3 of feature block fb = xfb(2 fi)
  constexpr int NAF = SQ ? 2 : 1;
  int offA0[NAF], offA1[NAF];
#pragma unroll
  for (int fi = 0; fi < NAF; ++fi) {
    const int cA = 4 * xfb(2 * fi) + 2 * (q & 1) + ((li & 3) >> 1);
    offA0[fi] = jX * DS + ((cA ^ row_swz<DS / 8>(jX)) << 3) + 4 * (li & 1);
    offA1[fi] = (jX + 4) * DS + ((cA ^ row_swz<DS / 8>(jX + 4)) << 3) + 4 * (li & 1);
  }
  //     B = G^T: samples 32 nb + 16 (q&1) + 4 (li&3) .. +3; swizzled chunk 4 (nb ^ (s>>2)) + (c ^ (s&3))
  //     for sample block nb = xsb(k) (k < NOB; further blocks of the same residue mod 4 by offset)
  const int cBl = 2 * (q & 1) + ((li & 3) >> 1);
  constexpr int NOBX = SQ ? 2 : NOB;
  int offB[2][NOBX];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const int sB = row_swz<MB / 8>(jX + 4 * w);
#pragma unroll
    for (int k = 0; k < NOBX; ++k)
      offB[w][k] = (jX + 4 * w) * MB + 32 * (xsb(k) ^ (sB >> 2)) + ((cBl ^ (sB & 3)) << 3) + 4 * (li & 1);
  }
  //   update: old weights of W row jb*32 + l32, features dblk*32 + 16u + 4hi (chunk 4 dblk + 2u) and
  //   + 8 (chunk 4 dblk + 2u + 1), 4 each at element 4 hi of the chunk
  const int sU = row_swz<DS / 8>(l32);
  int offUA[2], offUB[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    offUA[u] = l32 * DS + (((4 * dblk + 2 * u) ^ sU) << 3) + 4 * hi;
    offUB[u] = l32 * DS + (((4 * dblk + 2 * u + 1) ^ sU) << 3) + 4 * hi;
  }
  const int fU = dsl + dblk * 32;                              // the wave's first feature

  // Staging of the next tile through registers, one 16-byte chunk per item: items 0 .. GPT-1 are
  // G chunks (thread chunk ci = tid + c * NT is row ci / GCPR, chunk ci % GCPR: coalesced reads),
  // then WPT weight chunks (row ci / WCPR, 16-byte part ci % WCPR). The loads are spread over the
  // first half of a tile's MFMA slots and the LDS writes over the second half, so that neither a
  // burst of loads stalls the wave at the memory queue nor the wait for them sits between tiles.
  constexpr int NLD = GPT + WPT;
  i32x4_t gst[GPT], wst[WPT];
  auto load_item = [&](auto K, int tn) {
    constexpr int k = decltype(K)::value;
    if constexpr (k < GPT) {
      gst[k] = ((const i32x4_t*)(G + (int64_t)tn * TJ2 * MB))[tid + k * NT];
    } else {
      constexpr int c = k - GPT;
      const int ci = tid + c * NT, jr = ci / WCPR, p = ci % WCPR;
      if constexpr (WF == W_MXFP4_) {
        // 16 codes (8 bytes) and the scale byte of their 32-element block
        const int ro = (tn * TJ2 + jr) * rowbytes;
        const i32x2_t cd = __builtin_amdgcn_raw_buffer_load_b64(wres, ro + dsl / 2 + p * 8, 0, 0);
        const int sc = (int)__builtin_amdgcn_raw_buffer_load_b8(wres, ro + D / 2 + dsl / 32 + p / 2, 0, 0);
        wst[c] = i32x4_t{cd[0], cd[1], sc, 0};
      } else {
        wst[c] = buffer_load16(wres, (tn * TJ2 + jr) * rowbytes + dsl * ESZ + p * 16);
      }
    }
  };
  auto store_item = [&](auto K, uint16_t* gdst, int wb) {
    constexpr int k = decltype(K)::value;
    if constexpr (k < GPT) {
      // chunk ci of the tile's G blocks (lane (l, h) of half u of block (jb, sb)): label row
      // 32 jb + l, 16-byte sample chunk 4 sb + 2 u + h
      const int ci = tid + k * NT, cl = ci & 63, blk = ci >> 7;
      const int row = 32 * (blk / (MB / 32)) + (cl & 31);
      const int ch = 4 * (blk % (MB / 32)) + 2 * ((ci >> 6) & 1) + (cl >> 5);
      *(i32x4_t*)(gdst + row * MB + ((ch ^ row_swz<MB / 8>(row)) << 3)) = gst[k];
    } else {
      constexpr int c = k - GPT;
      const int ci = tid + c * NT, jr = ci / WCPR, p = ci % WCPR;
      const int sw = row_swz<DS / 8>(jr);
      uint16_t* row = &Ws[wb][jr * DS];
      if constexpr (WF == W_BF16_) {
        *(i32x4_t*)(row + ((p ^ sw) << 3)) = wst[c];
      } else if constexpr (WF == W_MXFP4_) {
        const float sc = e8m0_to_f32((uint32_t)wst[c][2]);
        const uint32_t w0 = (uint32_t)wst[c][0], w1 = (uint32_t)wst[c][1];
        *(i32x4_t*)(row + (((2 * p) ^ sw) << 3)) =
            i32x4_t{(int)fp4x2_to_bf16x2<0>(w0, sc), (int)fp4x2_to_bf16x2<1>(w0, sc),
                    (int)fp4x2_to_bf16x2<2>(w0, sc), (int)fp4x2_to_bf16x2<3>(w0, sc)};
        *(i32x4_t*)(row + (((2 * p + 1) ^ sw) << 3)) =
            i32x4_t{(int)fp4x2_to_bf16x2<0>(w1, sc), (int)fp4x2_to_bf16x2<1>(w1, sc),
                    (int)fp4x2_to_bf16x2<2>(w1, sc), (int)fp4x2_to_bf16x2<3>(w1, sc)};
      } else {
        uint32_t b[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) e4m3x4_to_bf16x4((uint32_t)wst[c][w], b[2 * w], b[2 * w + 1]);
        *(i32x4_t*)(row + (((2 * p) ^ sw) << 3)) = i32x4_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        *(i32x4_t*)(row + (((2 * p + 1) ^ sw) << 3)) = i32x4_t{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
      }
    }
  };

  f32x16_t accP[NJB];                          // previous tile's dW (this wave's label blocks)
  int tP = 0, wbP = 0;                         // previous tile and its W buffer
  // update phase PH of the wave's label blocks of tile tU (old weights in W buffer wsU, dW in accP)
  auto upd_args = [&](auto PH, UpdState& st, const uint16_t* wsU, int tU) {
    constexpr int ph = decltype(PH)::value, jl = ph / UPD_PHASES;
    const int jb = jb0 + jl;
    const int ro = (tU * TJ2 + jb * 32 + l32) * rowbytes;
    upd_phase<WF>(ph % UPD_PHASES, st, accP[jl], wsU + jb * 32 * DS, offUA, offUB, wres,
                  ro + (WF == W_MXFP4_ ? fU / 2 : fU * ESZ), ro + D / 2 + fU / 32,
                  ((uint64_t)(c0 + tU * TJ2 + jb * 32 + l32) * (uint64_t)D + (uint64_t)fU) >> 5, hi, lr, seed, step);
  };
  auto update = [&](int tU, int wbU) {         // the whole update of tile tU, in sequence
    UpdState st;
    static_for<0, NJB * UPD_PHASES>([&](auto PH) { upd_args(PH, st, Ws[wbU], tU); });
  };
  auto tile = [&](int t, int wb, auto gb, auto upd, auto pre, auto post) {
    constexpr bool UPD = decltype(upd)::value;
    constexpr int GB = decltype(gb)::value;    // G buffer of this tile (compile time)
    const int wbn = wb == 2 ? 0 : wb + 1;      // W buffer of tile t+1
    // the next tile (on the range's last tile, a repeat of a valid tile: the staging is then unused)
    const int tn = t + 1 < nt ? t + 1 : nt - 1;
    uint16_t* gnext = GB ? Gs0 : Gs1;
    __syncthreads();                           // tile t resident; iteration t-1 fully done
    if constexpr (NH == 2) static_for<0, NLD>([&](auto K) { load_item(K, tn); });
    pre(t);
    const uint16_t* gs = GB ? Gs1 : Gs0;
    const uint16_t* ws = Ws[wb];
    auto rdW = [&](int m) {                    // dW MFMA m: label block m % NJB, K step m / NJB
      const int jl = m % NJB, kk = m / NJB;
      return *(const s16x8_t*)(gs + offW[kk % NOW] + 16 * (kk - kk % NOW) + jl * 32 * MB);
    };
    auto rdXa = [&](int kx, int fi) {          // A of K step kx, feature block xfb(2 fi)
      return join(lds_read_tr16(ws + offA0[fi] + kx * 16 * DS), lds_read_tr16(ws + offA1[fi] + kx * 16 * DS));
    };
    auto rdXb = [&](int m) {                   // dX MFMA m: K step m / NBW, sample block nb0 + m % NBW
      const int kx = m / NBW, nb = m % NBW, k = nb % NOB, o = 32 * (nb - k) + kx * 16 * MB;
      return join(lds_read_tr16(gs + offB[0][k] + o), lds_read_tr16(gs + offB[1][k] + o));
    };
    auto rdXb2 = [&](int kx, int si) {         // B of K step kx, sample block xsb(si) (square blocking)
      return join(lds_read_tr16(gs + offB[0][si] + kx * 16 * MB), lds_read_tr16(gs + offB[1][si] + kx * 16 * MB));
    };
    UpdState st;
    const uint16_t* wsP = Ws[wbP];
    s16x8_t opW[NDW], opXb[NDX], opXa[KXN], opXa2[KXN][2], opXb2[KXN][2];
    f32x16_t accW[NJB];
#pragma unroll
    for (int jl = 0; jl < NJB; ++jl) accW[jl] = f32x16_t{};
    // operand reads of slot z (dW for even z, dX for odd z)
    auto fetch = [&](auto Z) {
      constexpr int z = decltype(Z)::value, m = z >> 1;
      if constexpr ((z & 1) == 0) {
        opW[m] = rdW(m);
      } else if constexpr (SQ) {
        // accumulator a = m % 4 of K step m / 4: (feature block a >> 1, sample block a & 1); each
        // fragment is read for the first MFMA that uses it
        constexpr int kx = m / 4, a = m % 4;
        if constexpr (a == 0) { opXa2[kx][0] = rdXa(kx, 0); opXb2[kx][0] = rdXb2(kx, 0); }
        else if constexpr (a == 1) opXb2[kx][1] = rdXb2(kx, 1);
        else if constexpr (a == 2) opXa2[kx][1] = rdXa(kx, 1);
      } else {
        if constexpr (m % NBW == 0) opXa[m / NBW] = rdXa(m / NBW, 0);
        opXb[m] = rdXb(m);
      }
    };
    static_for<0, PFS>(fetch);
    static_for<0, NSLOT>([&](auto Z) {
      constexpr int z = decltype(Z)::value, m = z >> 1;
      if constexpr (z + PFS < NSLOT) fetch(std::integral_constant<int, z + PFS>{});
      constexpr int HALF = NSLOT / 2;
      if constexpr (NH == 1)                   // loads over the first half, LDS writes over the second
        static_for<0, NLD>([&](auto K) {
          if constexpr (decltype(K)::value * HALF / NLD == z) load_item(K, tn);
          if constexpr (HALF + decltype(K)::value * HALF / NLD == z) store_item(K, gnext, wbn);
        });
      else                                     // (loads issued after the barrier) LDS writes over the last third
        static_for<0, NLD>([&](auto K) {
          constexpr int S0 = NSLOT - NSLOT / 3;
          if constexpr (S0 + decltype(K)::value * (NSLOT - S0) / NLD == z) store_item(K, gnext, wbn);
        });
      if constexpr ((z & 1) == 0) accW[m % NJB] = mfma_bf16(xT[m / NJB], opW[m], accW[m % NJB]);
      else if constexpr (SQ) accX[m % 4] = mfma_bf16(opXa2[m / 4][(m % 4) >> 1], opXb2[m / 4][m & 1], accX[m % 4]);
      else accX[m % NBW] = mfma_bf16(opXa[m / NBW], opXb[m], accX[m % NBW]);
      if constexpr (UPD) {
        // update phases ph with floor(ph * NSLOT / NPH) == z
        constexpr int NPH = NJB * UPD_PHASES;
        static_for<(z * NPH + NSLOT - 1) / NSLOT, ((z + 1) * NPH + NSLOT - 1) / NSLOT>(
            [&](auto PH) { upd_args(PH, st, wsP, tP); });
      }
      sched_fence();
    });
#pragma unroll
    for (int jl = 0; jl < NJB; ++jl) accP[jl] = accW[jl];
    post(t, wb);
    tP = t;
    wbP = wb;
  };

  // every range has a tile (the host launches at most as many ranges as the chunk has tiles), so
  // every slot of the first chunk is written
  if (t0 >= t1) return;
  {
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, 1>;
    static_for<0, NLD>([&](auto K) { load_item(K, t0); });
    sched_fence();
    init_acc();
    sched_fence();
    static_for<0, NLD>([&](auto K) { store_item(K, Gs0, 0); });
    if constexpr (NH == 1) {
      // one wave per SIMD: the previous tile's update is spread between this tile's MFMAs
      auto none = [](int) {};
      auto none2 = [](int, int) {};
      tile(t0, 0, G0{}, std::false_type{}, none, none2);
      int wb = 1;
      for (int t = t0 + 1; t < t1; t += 2) {
        tile(t, wb, G1{}, std::true_type{}, none, none2);
        wb = wb == 2 ? 0 : wb + 1;
        if (t + 1 < t1) {
          tile(t + 1, wb, G0{}, std::true_type{}, none, none2);
          wb = wb == 2 ? 0 : wb + 1;
        }
      }
      update(tP, wbP);
    } else {
      // two waves per SIMD (halves h = 0, 1 of a feature block) in complementary phases: half 0
      // updates its label block right after a tile's MFMAs, half 1 before the next tile's MFMAs, so
      // that on each SIMD the MFMAs of one wave overlap the update arithmetic of the other. The next
      // tile's staging loads are issued right after the barrier and written to LDS after the wave's
      // update (half 0) or late in its MFMA phase (half 1), so that an update phase and most of an
      // MFMA phase cover their latency.
      auto pre = [&](int t) { if (h == 1 && t > t0) update(t - 1, wbP); };
      auto post = [&](int t, int wbc) { if (h == 0) update(t, wbc); };
      int wb = 0;
      for (int t = t0; t < t1; t += 2) {
        tile(t, wb, G0{}, std::false_type{}, pre, post);
        wb = wb == 2 ? 0 : wb + 1;
        if (t + 1 < t1) {
          tile(t + 1, wb, G1{}, std::false_type{}, pre, post);
          wb = wb == 2 ? 0 : wb + 1;
        }
      }
      if (h == 1) update(tP, wbP);
    }
  }

  // the range's running dX partial back to its slot
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      *(f32x4_t*)pslot(nb, ig) =
          f32x4_t{accX[nb][4 * ig], accX[nb][4 * ig + 1], accX[nb][4 * ig + 2], accX[nb][4 * ig + 3]};
    }
}

// ------------------------------------------------------------------------------------------------
// forward + gradient with BF16 features stationary in registers (BF16 weights, 65-128 samples,
// D = 768)
// ------------------------------------------------------------------------------------------------
// The 8.6M-label head's shape, where the tiled forward re-stages every feature row for every tile.
// Four waves, one per SIMD, so that a lane has the whole register file: wave w holds samples
// 32 w .. 32 w + 31 as its MFMA A fragments of all 768 features (8 BF16 per 16-feature K step,
// 192 registers) and the work-group streams the chunk's weights through LDS in 32-label tiles
// (48 KiB each, row pitch 1,552 bytes: an odd number of 16-byte groups, so 16 consecutive rows'
// fragment reads fall on distinct banks), two buffers as in k_fwd_xs: tile t is loaded into
// registers at the start of iteration t - 1 and written to LDS at its end. Per tile a wave runs
// 48 MFMAs into one accumulator in K order and the gradient epilogue of its 32 x 32 block; one
// barrier per iteration; the positives of tile
// i + 1 are gathered into label bits during iteration i. Work-groups take tiles blockIdx.x,
// + gridDim.x, ...; tiles past the chunk read as zero, and the tiles cover whole 64-label
// backward tiles, so every G row the backward reads is written (zeros past the chunk).
constexpr int XB_TJ = 32;                                      // labels per tile

template <bool LOSS, bool ZOUT>
__global__ __launch_bounds__(256, 1) void k_fwd_xb(const uint8_t* __restrict__ W, const uint16_t* __restrict__ Xb,
                                                int D, int64_t c0, int clen,
                                                const uint32_t* __restrict__ tile_off,
                                                const uint32_t* __restrict__ bucket, int64_t bucket_cap,
                                                int B, uint16_t* __restrict__ G, int64_t gpitch,
                                                float* __restrict__ loss_part,
                                                float* __restrict__ Z, uint16_t* __restrict__ Gout,
                                                int64_t zpitch, int64_t zoff) {
  constexpr int MB = 128, D_ = 768, NK = D_ / 16;    // 48 K steps of the BF16 MFMA
  constexpr int RB = 2 * D_;                         // bytes per weight row
  constexpr int PITCH = RB + 16;
  static_assert((PITCH / 16) % 2 == 1, "an odd number of 16-byte groups per row");
  constexpr int PPR = RB / 16;                       // 16-byte parts per row
  constexpr int CPT = XB_TJ * PPR / 256;             // 16-byte chunks per thread and tile
  static_assert(CPT * 256 == XB_TJ * PPR, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) uint8_t Ws[2][XB_TJ * PITCH];
  __shared__ uint32_t ybits[4][XB_TJ * (MB / 32)];   // label-major: bit b & 31 of word [j][b >> 5]
  __shared__ float lred[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int bb = 32 * wave;                           // the wave's first sample
  // tiles of the chunk, rounded up to whole 64-label backward tiles: the backward reads G rows up
  // to the next multiple of 64, so those past the chunk are written too (as zeros)
  const int ntl = 2 * ((clen + 2 * XB_TJ - 1) / (2 * XB_TJ));
  const int nmy = ntl > (int)blockIdx.x ? (ntl - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  auto tile_of = [&](int i) { return (int)blockIdx.x + i * (int)gridDim.x; };
  (void)D;
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + c0 * (int64_t)RB, clen * RB);

  // chunk c of this thread: ci = tid + 256 c, row ci / PPR, part ci % PPR
  i32x4_t stg[CPT];
  auto wload = [&](int t, i32x4_t (&st)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + 256 * c, row = ci / PPR, part = ci % PPR;
      st[c] = buffer_load16(wres, (t * XB_TJ + row) * RB + part * 16);
    }
  };
  auto wstore = [&](int buf, const i32x4_t (&st)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + 256 * c, row = ci / PPR, part = ci % PPR;
      *(i32x4_t*)(&Ws[buf][row * PITCH + part * 16]) = st[c];
    }
  };
  // positives of tile t: quarter t & 3 of 128-label bucket tile c0 / 128 + t / 4 (c0 is a multiple
  // of 128)
  auto yclear = [&](int buf) {
    for (int i = tid; i < XB_TJ * (MB / 32); i += 256) ybits[buf][i] = 0u;
  };
  auto yscan = [&](int t, int buf) {
    const int64_t tb = c0 / TJ1 + (t >> 2);
    const uint32_t quarter = (uint32_t)(t & 3);
    const uint64_t e0 = tile_off[tb];
    const uint64_t e1 = tile_off[tb + 1] < (uint64_t)bucket_cap ? tile_off[tb + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 256) {
      const uint32_t v = bucket[e];
      const uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB && (jl >> 5) == quarter)
        atomicOr(&ybits[buf][(jl & (XB_TJ - 1)) * (MB / 32) + (b >> 5)], 1u << (b & 31));
    }
  };

  // prologue: tile 0, then the feature fragments, all in flight together; the tile's LDS writes
  // wait only for the tile loads (issued first), then tile 0's positives
  s16x8_t xf[NK];
  wload(tile_of(0), stg);
  {
    // (in the step preparation's fragment order: K step kk of this wave at (wave NK + kk) KiB; one
    // lane offset, the K step's in the instructions' scalar offsets)
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(Xb, MB * D_ * 2);
    const int xo = (wave * NK * 64 + lane) * 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) xf[kk] = __builtin_bit_cast(s16x8_t, buffer_load16(xres, xo, kk * 1024));
  }
  yclear(0); yclear(1); yclear(2);
  wstore(0, stg);
  __syncthreads();
  if (nmy > 0) yscan(tile_of(0), 0);
  __syncthreads();

  float lsum = 0.0f;
  for (int i = 0; i < nmy; ++i) {
    if (i + 1 < nmy) wload(tile_of(i + 1), stg);
    // the tile's 48 MFMAs, one chain in K order (the sums of the tiled forward and of the top-k
    // scans, so that a BF16 logit has the same bits whichever kernel computes it), each weight
    // fragment read from LDS two K steps ahead
    f32x16_t z = f32x16_t{};
    {
      const uint8_t* wb = &Ws[i & 1][l32 * PITCH + hi * 16];
      auto rd = [&](int kk) { return *(const s16x8_t*)(wb + kk * 32); };
      s16x8_t f[3];
      f[0] = rd(0); f[1] = rd(1);
      static_for<0, NK>([&](auto K) {
        constexpr int kk = decltype(K)::value;
        if constexpr (kk + 2 < NK) f[(kk + 2) % 3] = rd(kk + 2);
        z = mfma_bf16(xf[kk], f[kk % 3], z);
        sched_fence();
      });
    }
    {
      const int t = tile_of(i);
      const int jc = t * XB_TJ + l32;                 // label within the chunk
      const bool jvalid = jc < clen;
      const uint32_t yw = ybits[i & 3][l32 * (MB / 32) + wave];
      float gv[16];
      fwd_grad_block(z, yw, jvalid, bb, B, hi, gv);
      if constexpr (LOSS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bl = 8 * (r >> 2) + 4 * hi + (r & 3);
          if (jvalid && (bb + bl < B)) lsum += bce_loss(z[r], (yw >> bl) & 1u);
        }
      }
      if constexpr (ZOUT) {
        const int64_t lab = c0 + jc;
        const bool lok = jvalid && lab >= zoff;
        const int64_t base = (int64_t)(bb + 4 * hi) * zpitch + (lab - zoff);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + (r & 3);
          if (lok && bb + 4 * hi + rr < B) {
            const int64_t o = base + rr * zpitch;
            if (Z) Z[o] = z[r];
            if (Gout) Gout[o] = (uint16_t)f32_to_bf16_rne(gv[r]);
          }
        }
      }
      if constexpr (!ZOUT) fwd_store_block(gv, G, MB, jc, bb, lane);
    }
    if (i + 1 < nmy) wstore((i + 1) & 1, stg);
    if (i + 1 < nmy) yscan(tile_of(i + 1), (i + 1) & 3);
    yclear((i + 2) & 3);
    __syncthreads();
  }

  if constexpr (LOSS) {
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    if (tid == 0) loss_part[c0 / XB_TJ + blockIdx.x] = lred[0] + lred[1] + lred[2] + lred[3];
  }
}

// ------------------------------------------------------------------------------------------------
// chunk scheduler: per label chunk the forward + gradient kernel, then the backward + update kernel
// ------------------------------------------------------------------------------------------------
#define LAUNCH_CHECK() do { if (hipGetLastError() != hipSuccess) return ELMO_EHIP_; } while (0)

template <int MB, int WF>
int run_chunks(const StepArgs& a, const StepLayout& s, uint8_t* ws, hipStream_t st) {
  uint8_t* W = (uint8_t*)a.W;
  const uint8_t* Xf = WF == W_BF16_ ? ws + s.xb : ws + s.xq;
  uint16_t* Gc = (uint16_t*)(ws + s.g);
  const uint32_t* toff = (const uint32_t*)(ws + s.tile_off);
  const uint32_t* bucket = (const uint32_t*)(ws + s.bucket);
  float* part = (float*)(ws + s.part);
  float* lpart = (float*)(ws + s.loss);
  const int64_t l_end = a.l1;
  // the forward with the features stationary in registers where it is built (E4M3 and MXFP4 at 256
  // padded samples, D = 768); the tiled forward elsewhere
  constexpr bool XS_OK = MB == 256 && (WF == W_E4M3_ || WF == W_MXFP4_);
  const bool xs = XS_OK && (fwd_x_layout(MB, WF, a.D) == XLAY_XS_E4M3 || fwd_x_layout(MB, WF, a.D) == XLAY_XS_MX);
  // and for BF16 weights at 65-128 padded samples (the 8.6M-label head's shape)
  constexpr bool XB_OK = MB == 128 && WF == W_BF16_;
  const bool xb = XB_OK && fwd_x_layout(MB, WF, a.D) == XLAY_XB;
  for (int64_t c0 = a.l0; c0 < l_end; c0 += s.Cc) {
    const int clen = (int)((l_end - c0) < s.Cc ? (l_end - c0) : s.Cc);
    const int nt1 = (clen + TJ1 - 1) / TJ1;
    const int ntx = (clen + XS_TJ - 1) / XS_TJ;
    const int gx = ntx < s.cus ? ntx : s.cus;
    const int ntb = 2 * ((clen + 2 * XB_TJ - 1) / (2 * XB_TJ));   // (as the kernel counts its tiles)
    const int gb = ntb < s.cus ? ntb : s.cus;
    auto forward = [&](auto LOSS, auto ZOUT, float* Z, uint16_t* Gout, int64_t zpitch, int64_t zoff) {
      constexpr bool L_ = decltype(LOSS)::value, Z_ = decltype(ZOUT)::value;
      if constexpr (XS_OK) {
        if (xs) {
          hipLaunchKernelGGL((k_fwd_xs<WF, 12, L_, Z_>), dim3(gx), dim3(512), 0, st, W, ws + s.xq, a.D, c0, clen, toff,
                             bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, Z, Gout, zpitch, zoff);
          return;
        }
      }
      if constexpr (XB_OK) {
        if (xb) {
          hipLaunchKernelGGL((k_fwd_xb<L_, Z_>), dim3(gb), dim3(256), 0, st, W, (const uint16_t*)(ws + s.xb), a.D, c0,
                             clen, toff, bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, Z, Gout, zpitch, zoff);
          return;
        }
      }
      if constexpr (WF == W_MXFP4_) {
        hipLaunchKernelGGL((k_fwd_mx<MB, L_, Z_>), dim3(nt1), dim3(256), 0, st, W, Xf, a.D, c0, clen, toff, bucket,
                           a.nnz, a.B, Gc, (int64_t)MB, lpart, Z, Gout, zpitch, zoff);
      } else {
        hipLaunchKernelGGL((k_fwd_g<MB, WF, L_, Z_>), dim3(nt1), dim3(256), 0, st, W, Xf, a.D, c0, clen, toff,
                           bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, Z, Gout, zpitch, zoff);
      }
    };
    if (a.forward_only()) {
      forward(std::false_type{}, std::true_type{}, a.Z, a.Gout, a.zpitch, a.zoff);
      LAUNCH_CHECK();
      continue;
    }
    kt_begin(KT_FWD, st, clen);
    if (a.loss) forward(std::true_type{}, std::false_type{}, (float*)nullptr, (uint16_t*)nullptr, (int64_t)0, (int64_t)0);
    else forward(std::false_type{}, std::false_type{}, (float*)nullptr, (uint16_t*)nullptr, (int64_t)0, (int64_t)0);
    LAUNCH_CHECK();
    kt_end(KT_FWD, st);
    const int nt2 = (clen + TJ2 - 1) / TJ2;
    const int NR = nt2 < s.NR ? nt2 : s.NR;
    const int grid2 = 8 * ((NR * s.NS + 7) / 8);
    const int first = c0 == a.l0 && NR == s.NR;    // writes every partial slot: no zero fill needed
    kt_begin(KT_BWD, st, clen);
    // two waves per feature block (complementary phases) at 64 and 256 samples; at 128 samples the
    // one-wave form, with the update spread between the next tile's MFMAs, is faster (measured:
    // 0.193 vs 0.217 ms per 262k-label BF16 chunk), and at 32 it is the only form
    constexpr int NH = MB == 64 || MB == 256 ? 2 : 1;
    if (s.DS == 128)
      hipLaunchKernelGGL((k_bwd_update<MB, WF, 128, NH>), dim3(grid2), dim3(256 * NH), 0, st, W, a.D, c0, clen,
                         (const uint16_t*)(ws + s.xbt), Gc, part, NR, s.NS, a.lr, a.seed, a.step, first);
    else
      hipLaunchKernelGGL((k_bwd_update<MB, WF, 64, NH>), dim3(grid2), dim3(128 * NH), 0, st, W, a.D, c0, clen,
                         (const uint16_t*)(ws + s.xbt), Gc, part, NR, s.NS, a.lr, a.seed, a.step, first);
    LAUNCH_CHECK();
    kt_end(KT_BWD, st);
  }
  return ELMO_OK_;
}

#if defined(ELMO_MB) && defined(ELMO_WF)
template int run_chunks<ELMO_MB, ELMO_WF>(const StepArgs&, const StepLayout&, uint8_t*, hipStream_t);
#endif

}  // namespace elmo
