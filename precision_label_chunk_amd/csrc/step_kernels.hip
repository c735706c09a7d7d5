// The chunked, fused XMC classifier-head training step on gfx950.
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
// Label handling, X preparation and the final dX reduction are small kernels around them.
#include "step_kernels.hpp"

#include <type_traits>
#include <vector>

#include "fwd_tile.hpp"
#include "mfma.hpp"
#include "numerics.hpp"

namespace elmo {

// ------------------------------------------------------------------------------------------------
// small kernels
// ------------------------------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Label bucketing by 128-label tile: counts, exclusive offsets, then the bucket entries
// (sample << 16 | label within the tile). A work-group handles LSPB samples, one wave per sample at
// a time; counts of the first LHOT tiles (where a skewed label law concentrates its mass) are first
// gathered in LDS and added to the global counters once per work-group, so a popular tile costs one
// global atomic per work-group instead of one per occurrence.
constexpr int LSPB = 16, LHOT = 4096;

// validate sample b's CSR row (flags) and return its clamped entry range
__device__ __forceinline__ void label_row(const int32_t* __restrict__ row_ptr, int b, int B, int64_t nnz,
                                          uint32_t* __restrict__ flags, bool check, int64_t& r0, int64_t& r1) {
  r0 = row_ptr[b]; r1 = row_ptr[b + 1];
  if (check) {
    const bool bad = r0 < 0 || r1 < r0 || r1 > nnz || (b == 0 && r0 != 0) || (b == B - 1 && r1 != nnz);
    if (bad) atomicOr(flags, ELMO_FLAG_ROW_PTR_);
  }
  r0 = r0 < 0 ? 0 : (r0 > nnz ? nnz : r0);
  r1 = r1 < r0 ? r0 : (r1 > nnz ? nnz : r1);
}

__global__ __launch_bounds__(256) void k_label_count(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ ids,
                                                     int B, int64_t nnz, int64_t L, int64_t ntiles,
                                                     uint32_t* __restrict__ tile_cnt, uint32_t* __restrict__ flags) {
  __shared__ uint32_t h[LHOT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = tid; t < LHOT; t += 256) h[t] = 0u;
  __syncthreads();
  const int b0 = blockIdx.x * LSPB, b1 = b0 + LSPB < B ? b0 + LSPB : B;
  for (int b = b0 + wave; b < b1; b += 4) {
    int64_t r0, r1;
    label_row(row_ptr, b, B, nnz, flags, lane == 0, r0, r1);
    for (int64_t i = r0 + lane; i < r1; i += 64) {
      const int32_t id = ids[i];
      if (id < 0 || id >= L) { atomicOr(flags, ELMO_FLAG_LABEL_RANGE_); continue; }
      const int t = id / TJ1;
      if (t < LHOT) atomicAdd(&h[t], 1u);
      else atomicAdd(&tile_cnt[t], 1u);
    }
  }
  __syncthreads();
  for (int t = tid; t < LHOT && t < ntiles; t += 256)
    if (h[t]) atomicAdd(&tile_cnt[t], h[t]);
}

// exclusive scan of the per-tile counts by one work-group of 1024 threads, in segments of LSEG
// counts staged in LDS (coalesced loads and stores): thread t scans its run of LSEG/1024
// consecutive counts, the run sums are scanned across the work-group, a running carry joins the
// segments; cnt becomes the scatter cursor and off[ntiles] the total. Count i of a segment sits at
// LDS word i + i / LRUN (a pad word after each run keeps the runs' reads on distinct banks).
constexpr int LSEG = 32768, LRUN = LSEG / 1024;
__global__ __launch_bounds__(1024) void k_label_scan(uint32_t* __restrict__ cnt, uint32_t* __restrict__ off,
                                                     int64_t ntiles) {
  __shared__ uint32_t seg[LSEG + LSEG / LRUN];
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t carry = 0;
  for (int64_t base = 0; base < ntiles; base += LSEG) {
    const int64_t n = ntiles - base < LSEG ? ntiles - base : LSEG;
#pragma unroll
    for (int k = 0; k < LRUN; ++k) {
      const int i = tid + 1024 * k;
      seg[i + i / LRUN] = i < n ? cnt[base + i] : 0u;
    }
    __syncthreads();
    uint32_t tsum = 0;
#pragma unroll 8
    for (int k = 0; k < LRUN; ++k) tsum += seg[tid * (LRUN + 1) + k];
    // inclusive scan of the run sums within the wave, then across the 16 waves
    uint32_t x = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t wpre = carry, total = carry;
    for (int w = 0; w < 16; ++w) {
      const uint32_t t = wsum[w];
      if (w < wave) wpre += t;
      total += t;
    }
    uint32_t run = wpre + x - tsum;             // exclusive prefix of this thread's run
#pragma unroll 8
    for (int k = 0; k < LRUN; ++k) {
      const uint32_t v = seg[tid * (LRUN + 1) + k];
      seg[tid * (LRUN + 1) + k] = run;
      run += v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < LRUN; ++k) {
      const int i = tid + 1024 * k;
      if (i < n) { off[base + i] = seg[i + i / LRUN]; cnt[base + i] = seg[i + i / LRUN]; }
    }
    carry = total;
    __syncthreads();                            // seg and wsum free for the next segment
  }
  if (tid == 0) off[ntiles] = carry;
}

// bucket capacity is nnz: with a malformed row_ptr (overlapping rows) entries beyond it are dropped
__global__ __launch_bounds__(256) void k_label_scatter(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ ids,
                                                       int B, int64_t nnz, int64_t L, int64_t ntiles,
                                                       uint32_t* __restrict__ cursor, uint32_t* __restrict__ bucket) {
  __shared__ uint32_t h[LHOT];                    // counts of this work-group's entries, then its cursors
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = tid; t < LHOT; t += 256) h[t] = 0u;
  __syncthreads();
  const int b0 = blockIdx.x * LSPB, b1 = b0 + LSPB < B ? b0 + LSPB : B;
  for (int b = b0 + wave; b < b1; b += 4) {
    int64_t r0, r1;
    label_row(row_ptr, b, B, nnz, nullptr, false, r0, r1);
    for (int64_t i = r0 + lane; i < r1; i += 64) {
      const int32_t id = ids[i];
      if (id >= 0 && id < L && id / TJ1 < LHOT) atomicAdd(&h[id / TJ1], 1u);
    }
  }
  __syncthreads();
  for (int t = tid; t < LHOT && t < ntiles; t += 256)    // reserve this work-group's range per tile
    if (h[t]) h[t] = atomicAdd(&cursor[t], h[t]);
  __syncthreads();
  for (int b = b0 + wave; b < b1; b += 4) {
    int64_t r0, r1;
    label_row(row_ptr, b, B, nnz, nullptr, false, r0, r1);
    for (int64_t i = r0 + lane; i < r1; i += 64) {
      const int32_t id = ids[i];
      if (id < 0 || id >= L) continue;
      const int t = id / TJ1;
      const uint32_t pos = t < LHOT ? atomicAdd(&h[t], 1u) : atomicAdd(&cursor[t], 1u);
      if (pos < (uint64_t)nnz) bucket[pos] = ((uint32_t)b << 16) | (uint32_t)(id % TJ1);
    }
  }
}

// zero-padded BF16 copy of X ([MB][D]) and, in FP8 mode, its E4M3-RNE cast for the forward MFMA
__global__ void k_prep_x(const uint16_t* __restrict__ X, int B, int D, int MB, uint16_t* __restrict__ Xb,
                         uint8_t* __restrict__ Xq, uint16_t* __restrict__ XbT) {
  const int64_t n = (int64_t)MB * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t v = (i / D) < B ? X[i] : 0u;
    Xb[i] = (uint16_t)v;
    if (Xq) Xq[i] = (uint8_t)f32_to_e4m3_rne_sat(bf16_to_f32(v));
    // the feature-major copy XbT[d][b] (element i of it: d = i / MB, b = i % MB)
    const int64_t d = i / MB, b = i % MB;
    XbT[i] = b < B ? X[b * D + d] : (uint16_t)0;
  }
}

// dX[b][d] = sum over label ranges r (fixed order) of the FP32 partials. A range's partial holds
// the backward's 32 x 32 dX^T accumulator blocks: element p = (((fb * NB + sb) * 4 + ig) * 64 +
// lane) * 4 + e (feature block fb, sample block sb) is register i = 4 ig + e of that lane, feature
// 32 fb + 8 ig + 4 (lane / 32) + e of sample 32 sb + lane % 32.
__global__ void k_dx_reduce(const float* __restrict__ part, int NR, int MB, int D, int B, float* __restrict__ dX) {
  const int64_t n = (int64_t)MB * D;
  const int NB = MB / 32;
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < n; p += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(p & 3), lane = (int)((p >> 2) & 63), ig = (int)((p >> 8) & 3);
    const int64_t blk = p >> 10;
    const int sb = (int)(blk % NB), fb = (int)(blk / NB);
    const int b = 32 * sb + (lane & 31);
    if (b >= B) continue;
    const int d = 32 * fb + 8 * ig + 4 * (lane >> 5) + e;
    float s = 0.0f;
#pragma unroll 8
    for (int r = 0; r < NR; ++r) s += part[(int64_t)r * n + p];
    dX[(int64_t)b * D + d] = s;
  }
}

// summed loss: per-tile FP32 partials added in binary64 in a fixed order
__global__ __launch_bounds__(256) void k_loss_reduce(const float* __restrict__ lp, int64_t n, float* __restrict__ out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)lp[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)red[0];
}

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
    if (__builtin_amdgcn_ballot_w64(m > 2.0f) == 0) {
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

// Packing pairs to BF16 and swapping register groups 1 <-> 0 and 3 <-> 2 across the lane halves
// leaves 8 consecutive samples per lane and group pair, written with one 16-byte store each into
// the label's row `grow` of the label-major chunk buffer G[label][sample].
__device__ __forceinline__ void fwd_store_block(const float (&gv)[16], uint16_t* grow, int bb, int hi) {
  uint32_t pk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(gv[2 * k], gv[2 * k + 1]);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * u], pk[4 * u + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * u + 1], pk[4 * u + 3], false, false);
    const i32x4_t out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    *(i32x4_t*)(grow + bb + 16 * u + 8 * hi) = out;
  }
}

// The same 16-byte pieces into a wave's LDS staging rows instead (row `lrow`, byte column c0b of
// the block's first sample): the rows then go out as whole 128-byte segments.
__device__ __forceinline__ void fwd_stage_block(const float (&gv)[16], uint8_t* lrow, int c0b, int hi) {
  uint32_t pk[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(gv[2 * k], gv[2 * k + 1]);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * u], pk[4 * u + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * u + 1], pk[4 * u + 3], false, false);
    const i32x4_t out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
    *(i32x4_t*)(lrow + c0b + 32 * u + 16 * hi) = out;
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

  // epilogue: gradient straight from the accumulators, block by block. With 128 or 256 samples
  // each wave's rows of G (CW = 64 labels) are staged in LDS (free after the K loop) 64 samples at
  // a time, so that every row leaves as one whole 128-byte segment instead of 16-byte pieces of
  // 32 rows.
  constexpr bool GST = MB >= 128 && !ZOUT;
  constexpr int GSP = 144;                     // staging row pitch (bytes): 16 rows per bank cycle
  uint8_t* gst = smem + wave * (CW * GSP);
  float lsum = 0.0f;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
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
      if constexpr (GST) fwd_stage_block(gv, gst + (ni * 32 + l32) * GSP, (mi & 1) * 64, hi);
      else if constexpr (!ZOUT) fwd_store_block(gv, G + (int64_t)(jbase + jl) * gpitch, bb, hi);
    }
    if constexpr (GST) {
      if (mi & 1) {                            // 64 samples of the wave's CW rows staged
        const int sb0 = wb * RW + (mi - 1) * 32;
#pragma unroll
        for (int k = 0; k < CW / 8; ++k) {
          const int row = k * 8 + (lane >> 3);
          const i32x4_t v = *(const i32x4_t*)(gst + row * GSP + (lane & 7) * 16);
          *(i32x4_t*)(G + (int64_t)(jbase + wj * CW + row) * gpitch + sb0 + (lane & 7) * 8) = v;
        }
      }
    }
  }
  if constexpr (LOSS) {
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) lred[wave] = lsum;
    __syncthreads();
    if (tid == 0) loss_part[tg] = ((lred[0] + lred[1]) + lred[2]) + lred[3];
  }
}

// ------------------------------------------------------------------------------------------------
// backward + fused update over one d-slice and one label range of the chunk
// ------------------------------------------------------------------------------------------------
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
// p = 0..7), feature 16u + 8 (p >> 2) + 4 hi + (p & 3) of the 32: for each u the 8 elements of one
// RNG block (block 4 grp + 2u + hi, positions p in order, grp the index of the row's 32-element
// group), which the lane updates with one Philox block: t = fmaf(-lr, dW, w), hardware stochastic
// rounding. Swapping the packed results of block 1 of lane half 0 with those of block 0 of lane
// half 1 leaves each lane the 16 consecutive features 16 hi .. 16 hi + 15 of its label, stored in
// 16-byte pieces. The work is cut into UPD_PHASES phases so that it can be spread between MFMAs:
// 0 the RNG counters, 1..10 the Philox rounds (these RNG_PHASES need no dW), 11 old-weight reads,
// 12..19 two weights each (rounding and packing), 20 the exchange and the stores.
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
};

template <int WF>
__device__ __forceinline__ void upd_phase(int p, UpdState& st, const f32x16_t& acc, const uint16_t* ow,
                                          const int (&owa)[2], const int (&owb)[2], __amdgpu_buffer_rsrc_t wres,
                                          int roff, uint64_t grp, int hi, float lr, uint64_t seed, uint64_t step) {
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
  if (p == 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) st.c[u] = philox_counter(4 * grp + 2 * u + hi, step);
  } else if (p <= 10) {
    const uint32_t k0 = philox_key0(seed, p - 1), k1 = philox_key1(seed, p - 1);
    philox_round2(st.c[0], st.c[1], k0, k1);
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

// Work-group: NH * DS/32 waves. The NH waves of feature block fb own the 32 features
// [dsl + 32 fb, +32) of the slice and share the two backward contractions of every tile; with
// NH = 2 (two waves per SIMD for DS = 128, so that one wave's update arithmetic fills the other's
// MFMA and LDS waits) wave half h computes dW of label block h over all samples and dX of sample
// half h over all the tile's labels:
//   dW^T[d][j]  = sum_b X^T[d][b] G[b][j]      2/NH 32-label blocks, K = MB samples  (MB/8/NH MFMAs)
//   dX^T[d][b] += sum_j W^T[d][j] G^T[j][b]    MB/32/NH sample blocks, K = 64 labels (MB/8/NH MFMAs)
// with A = stationary X^T fragments in registers (dW), B = G rows by ds_read_b128 (dW), and
// A = W^T, B = G^T by ds_read_b64_tr_b16 (dX). Per 64-label tile t:
//   G tile  [64][MB] BF16 (label-major, as the forward kernel writes it), double buffered in two
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
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
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
  constexpr int STAGE_MODE = 2;
  constexpr int GTE = TJ2 * MB;                // G tile elements
  constexpr int GCPR = MB / 8;                 // 16-byte chunks per G row
  constexpr int GPT = TJ2 * GCPR / NT;         // G chunks per thread
  constexpr int WCPR = DS * ESZ / 16;          // 16-byte global W chunks per tile row
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
  const int rowbytes = D * ESZ;
  // the chunk's weight rows: rows past the chunk's end (the ragged last tile) load as zero and
  // drop their stores
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + c0 * (int64_t)rowbytes, clen * rowbytes);
  const int jb0 = NH == 2 ? h : 0;             // first label block of this wave
  const int nb0 = h * NBW;                     // first sample block of this wave

  // stationary X^T fragments of this wave's 32 features: lane (d, 8 samples), from the
  // feature-major copy XbT[d][b]
  s16x8_t xT[KK];
  {
    const int d = dsl + dblk * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) xT[kk] = *(const s16x8_t*)(XbT + (int64_t)d * MB + kk * 16 + hi * 8);
  }
  // dX^T accumulators, starting from this range's running partial sum (a fixed slot per range:
  // deterministic; zero in the step's first chunk, where every slot has a range), read here under
  // the first tile's staging and stored back at the end. The partial keeps the accumulators' own
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
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const f32x4_t o = first ? f32x4_t{} : *(const f32x4_t*)pslot(nb, ig);
      accX[nb][4 * ig] = o[0]; accX[nb][4 * ig + 1] = o[1]; accX[nb][4 * ig + 2] = o[2]; accX[nb][4 * ig + 3] = o[3];
    }

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
      wst[c] = buffer_load16(wres, (tn * TJ2 + jr) * rowbytes + dsl * ESZ + p * 16);
    }
  };
  auto store_item = [&](auto K, uint16_t* gdst, int wb) {
    constexpr int k = decltype(K)::value;
    if constexpr (k < GPT) {
      const int ci = tid + k * NT, row = ci / GCPR, ch = ci % GCPR;
      *(i32x4_t*)(gdst + row * MB + ((ch ^ row_swz<MB / 8>(row)) << 3)) = gst[k];
    } else {
      constexpr int c = k - GPT;
      const int ci = tid + c * NT, jr = ci / WCPR, p = ci % WCPR;
      const int sw = row_swz<DS / 8>(jr);
      uint16_t* row = &Ws[wb][jr * DS];
      if constexpr (WF == W_BF16_) {
        *(i32x4_t*)(row + ((p ^ sw) << 3)) = wst[c];
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
    upd_phase<WF>(ph % UPD_PHASES, st, accP[jl], wsU + jb * 32 * DS, offUA, offUB, wres,
                  (tU * TJ2 + jb * 32 + l32) * rowbytes + fU * ESZ,
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
    if constexpr (NH == 2 && STAGE_MODE != 0) static_for<0, NLD>([&](auto K) { load_item(K, tn); });
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
      if constexpr (NH == 1 || STAGE_MODE == 0)
        static_for<0, NLD>([&](auto K) {
          if constexpr (decltype(K)::value * HALF / NLD == z) load_item(K, tn);
          if constexpr (HALF + decltype(K)::value * HALF / NLD == z) store_item(K, gnext, wbn);
        });
      else if constexpr (STAGE_MODE >= 2)      // LDS writes spread over the slots from S0 on
        static_for<0, NLD>([&](auto K) {
          constexpr int S0 = STAGE_MODE == 2 ? NSLOT - NSLOT / 3 : HALF;
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
    if constexpr (NH == 2 && STAGE_MODE == 1) static_for<0, NLD>([&](auto K) { store_item(K, gnext, wbn); });
    tP = t;
    wbP = wb;
  };

  if (t0 < t1) {
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, 1>;
    static_for<0, NLD>([&](auto K) { load_item(K, t0); });
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
// host side: optional kernel timing, workspace layout, chunk scheduler, launches
// ------------------------------------------------------------------------------------------------
namespace {
struct KTRec { int kind; int64_t labels; hipEvent_t a, b; };
struct KTState {
  int on = 0;
  std::vector<KTRec> recs;      // pending launches (events reused through `pool`)
  std::vector<hipEvent_t> pool;
};
KTState& kt() { static KTState s; return s; }
hipEvent_t kt_event() {
  KTState& s = kt();
  if (!s.pool.empty()) { hipEvent_t e = s.pool.back(); s.pool.pop_back(); return e; }
  // timing only: no system-scope fence (cache writeback and invalidation) when the event is recorded,
  // which would otherwise add its cost between the launches it brackets
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void kernel_timing_enable(int on) { kt().on = on; }

void kt_begin(int kind, hipStream_t st, int64_t labels) {
  KTState& s = kt();
  if (!s.on) return;
  KTRec r{kind, labels, kt_event(), kt_event()};
  if (!r.a || !r.b) return;
  hipEventRecord(r.a, st);
  s.recs.push_back(r);
}

void kt_end(int kind, hipStream_t st) {
  KTState& s = kt();
  if (!s.on || s.recs.empty() || s.recs.back().kind != kind) return;
  hipEventRecord(s.recs.back().b, st);
}

int kernel_timing_read(double* ms, int64_t* launches, double* labels) {
  KTState& s = kt();
  for (int k = 0; k < 2; ++k) { ms[k] = 0.0; launches[k] = 0; labels[k] = 0.0; }
  int rc = ELMO_OK_;
  for (const KTRec& r : s.recs) {
    float t = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) rc = ELMO_EHIP_;
    ms[r.kind] += t; launches[r.kind] += 1; labels[r.kind] += (double)r.labels;
    s.pool.push_back(r.a); s.pool.push_back(r.b);
  }
  s.recs.clear();
  return rc;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int padded_batch(int B) { return B <= 32 ? 32 : B <= 64 ? 64 : B <= 128 ? 128 : 256; }

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

StepLayout step_layout(int B, int D, int64_t L, int64_t chunk, int wdtype, int64_t max_nnz) {
  StepLayout s{};
  s.MB = padded_batch(B);
  s.DS = (D % 128 == 0) ? 128 : 64;
  s.NS = D / s.DS;
  int64_t Lr = (L + TJ1 - 1) / TJ1 * TJ1;
  int64_t c = chunk - chunk % TJ1;
  if (c < TJ1) c = TJ1;
  if (c > Lr) c = Lr;
  // chunk-relative 32-bit byte offsets into the chunk's weight rows (one tile of slack)
  const int64_t rb = (int64_t)D * (wdtype == W_E4M3_ ? 1 : 2);
  const int64_t cmax = ((int64_t)0x7fffffff / rb - TJ1) / TJ1 * TJ1;
  if (c > cmax) c = cmax;
  s.Cc = c;
  s.ntiles = (L + TJ1 - 1) / TJ1;
  // backward work-groups hold a whole CU (LDS and registers): at most as many (range, slice)
  // work-groups as CUs, so the launch is one round; they are laid out XCD-major (see the kernel)
  int64_t nt2 = (c + TJ2 - 1) / TJ2;
  s.cus = device_cus();
  int cap = s.cus / s.NS;
  if (cap < 1) cap = 1;
  s.NR = (int)(nt2 < cap ? nt2 : cap);
  size_t off = 0;
  const size_t A = 256;
  s.flags = off;    off = align_up(off + 64, A);
  s.tile_cnt = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.tile_off = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.bucket = off;   off = align_up(off + 4 * (size_t)(max_nnz > 0 ? max_nnz : 1), A);
  s.xb = off;       off = align_up(off + 2 * (size_t)s.MB * D, A);
  s.xq = off;       off = align_up(off + (wdtype == W_E4M3_ ? (size_t)s.MB * D : 0), A);
  s.xbt = off;      off = align_up(off + 2 * (size_t)s.MB * D, A);
  s.g = off;        off = align_up(off + 2 * (size_t)s.MB * (size_t)s.Cc, A);
  s.part = off;     off = align_up(off + 4 * (size_t)s.NR * s.MB * D, A);
  s.loss = off;     off = align_up(off + 4 * (size_t)s.ntiles, A);
  s.total = off;
  return s;
}

#define LAUNCH_CHECK() do { if (hipGetLastError() != hipSuccess) return ELMO_EHIP_; } while (0)

template <int MB, int WF>
static int run_chunks(const StepArgs& a, const StepLayout& s, uint8_t* ws, hipStream_t st) {
  uint8_t* W = (uint8_t*)a.W;
  const uint8_t* Xf = WF == W_BF16_ ? ws + s.xb : ws + s.xq;
  uint16_t* Gc = (uint16_t*)(ws + s.g);
  const uint32_t* toff = (const uint32_t*)(ws + s.tile_off);
  const uint32_t* bucket = (const uint32_t*)(ws + s.bucket);
  float* part = (float*)(ws + s.part);
  float* lpart = (float*)(ws + s.loss);
  const int64_t l_end = a.l1;
  for (int64_t c0 = a.l0; c0 < l_end; c0 += s.Cc) {
    const int clen = (int)((l_end - c0) < s.Cc ? (l_end - c0) : s.Cc);
    const int nt1 = (clen + TJ1 - 1) / TJ1;
    if (a.forward_only()) {
      hipLaunchKernelGGL((k_fwd_g<MB, WF, false, true>), dim3(nt1), dim3(256), 0, st, W, Xf, a.D, c0, clen,
                         toff, bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, a.Z, a.Gout, a.zpitch, a.zoff);
      LAUNCH_CHECK();
      continue;
    }
    kt_begin(KT_FWD, st, clen);
    if (a.loss)
      hipLaunchKernelGGL((k_fwd_g<MB, WF, true, false>), dim3(nt1), dim3(256), 0, st, W, Xf, a.D, c0, clen,
                         toff, bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, (float*)nullptr, (uint16_t*)nullptr, (int64_t)0, (int64_t)0);
    else
      hipLaunchKernelGGL((k_fwd_g<MB, WF, false, false>), dim3(nt1), dim3(256), 0, st, W, Xf, a.D, c0, clen,
                         toff, bucket, a.nnz, a.B, Gc, (int64_t)MB, lpart, (float*)nullptr, (uint16_t*)nullptr, (int64_t)0, (int64_t)0);
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

int run_step(const StepArgs& a, const StepLayout& s, void* workspace, hipStream_t st) {
  uint8_t* ws = (uint8_t*)workspace;
  uint32_t* flags = (uint32_t*)(ws + s.flags);
  uint32_t* cnt = (uint32_t*)(ws + s.tile_cnt);
  uint32_t* off = (uint32_t*)(ws + s.tile_off);
  // zero flags, tile counts and (for a training step) the dX partial sums
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, st, flags, (int64_t)16, 0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(256), 0, st, cnt, s.ntiles + 1, 0u);
  LAUNCH_CHECK();
  if (!a.forward_only()) {
    // the first chunk stores all partial slots unless it has fewer label ranges than there are slots
    const int64_t clen0 = (a.l1 - a.l0) < s.Cc ? (a.l1 - a.l0) : s.Cc;
    if ((clen0 + TJ2 - 1) / TJ2 < s.NR) {
      hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, st, (uint32_t*)(ws + s.part),
                         (int64_t)s.NR * s.MB * a.D, 0u);
      LAUNCH_CHECK();
    }
  }
  const int lblocks = (a.B + LSPB - 1) / LSPB;
  if (a.B > 0 && a.row_ptr) {
    hipLaunchKernelGGL(k_label_count, dim3(lblocks), dim3(256), 0, st, a.row_ptr, a.ids, a.B, a.nnz, a.L, s.ntiles,
                       cnt, flags);
    LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_label_scan, dim3(1), dim3(1024), 0, st, cnt, off, s.ntiles);
  LAUNCH_CHECK();
  if (a.B > 0 && a.row_ptr && a.nnz > 0) {
    hipLaunchKernelGGL(k_label_scatter, dim3(lblocks), dim3(256), 0, st, a.row_ptr, a.ids, a.B, a.nnz, a.L,
                       s.ntiles, cnt, (uint32_t*)(ws + s.bucket));
    LAUNCH_CHECK();
  }
  {
    const int64_t n = (int64_t)s.MB * a.D;
    const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_prep_x, dim3(blocks), dim3(256), 0, st, (const uint16_t*)a.X, a.B, a.D, s.MB,
                       (uint16_t*)(ws + s.xb), a.wdtype == W_E4M3_ ? ws + s.xq : (uint8_t*)nullptr,
                       (uint16_t*)(ws + s.xbt));
    LAUNCH_CHECK();
  }
  int rc;
  const int MB = s.MB;
  if (a.wdtype == W_BF16_) {
    rc = MB == 32 ? run_chunks<32, W_BF16_>(a, s, ws, st) : MB == 64 ? run_chunks<64, W_BF16_>(a, s, ws, st)
       : MB == 128 ? run_chunks<128, W_BF16_>(a, s, ws, st) : run_chunks<256, W_BF16_>(a, s, ws, st);
  } else {
    rc = MB == 32 ? run_chunks<32, W_E4M3_>(a, s, ws, st) : MB == 64 ? run_chunks<64, W_E4M3_>(a, s, ws, st)
       : MB == 128 ? run_chunks<128, W_E4M3_>(a, s, ws, st) : run_chunks<256, W_E4M3_>(a, s, ws, st);
  }
  if (rc != ELMO_OK_ || a.forward_only()) return rc;
  {
    const int64_t n = (int64_t)s.MB * a.D;
    const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(k_dx_reduce, dim3(blocks), dim3(256), 0, st, (const float*)(ws + s.part), s.NR, s.MB,
                       a.D, a.B, a.dX);
    LAUNCH_CHECK();
  }
  if (a.loss) {
    hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(256), 0, st, (const float*)(ws + s.loss), s.ntiles, a.loss);
    LAUNCH_CHECK();
  }
  return ELMO_OK_;
}

}  // namespace elmo
