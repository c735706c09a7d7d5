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

// one block per sample: validate its CSR row and count its labels per 128-label tile
__global__ void k_label_count(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ ids,
                              int B, int64_t nnz, int64_t L, uint32_t* __restrict__ tile_cnt,
                              uint32_t* __restrict__ flags) {
  const int b = blockIdx.x;
  int64_t r0 = row_ptr[b], r1 = row_ptr[b + 1];
  if (threadIdx.x == 0) {
    bool bad = r0 < 0 || r1 < r0 || r1 > nnz || (b == 0 && r0 != 0) || (b == B - 1 && r1 != nnz);
    if (bad) atomicOr(flags, ELMO_FLAG_ROW_PTR_);
  }
  r0 = r0 < 0 ? 0 : (r0 > nnz ? nnz : r0);
  r1 = r1 < r0 ? r0 : (r1 > nnz ? nnz : r1);
  for (int64_t i = r0 + threadIdx.x; i < r1; i += blockDim.x) {
    int32_t id = ids[i];
    if (id < 0 || id >= L) { atomicOr(flags, ELMO_FLAG_LABEL_RANGE_); continue; }
    atomicAdd(&tile_cnt[id / TJ1], 1u);
  }
}

// exclusive scan of the per-tile counts (one block of 1024 threads); cnt becomes the scatter cursor
__global__ __launch_bounds__(1024) void k_label_scan(uint32_t* __restrict__ cnt, uint32_t* __restrict__ off,
                                                     int64_t ntiles) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t seg = (ntiles + 1023) / 1024;
  const int64_t a = tid * seg, e = (a + seg < ntiles) ? a + seg : ntiles;
  uint32_t s = 0;
  for (int64_t i = a; i < e; ++i) s += cnt[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {      // inclusive Hillis-Steele scan
    uint32_t v = tid >= o ? part[tid - o] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint32_t run = tid ? part[tid - 1] : 0u;
  for (int64_t i = a; i < e; ++i) {
    uint32_t c = cnt[i];
    off[i] = run;
    cnt[i] = run;
    run += c;
  }
  if (tid == 1023) off[ntiles] = part[1023];
}

// bucket capacity is nnz: with a malformed row_ptr (overlapping rows) entries beyond it are dropped
__global__ void k_label_scatter(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ ids,
                                int64_t nnz, int64_t L, uint32_t* __restrict__ cursor,
                                uint32_t* __restrict__ bucket) {
  const int b = blockIdx.x;
  int64_t r0 = row_ptr[b], r1 = row_ptr[b + 1];
  r0 = r0 < 0 ? 0 : (r0 > nnz ? nnz : r0);
  r1 = r1 < r0 ? r0 : (r1 > nnz ? nnz : r1);
  for (int64_t i = r0 + threadIdx.x; i < r1; i += blockDim.x) {
    int32_t id = ids[i];
    if (id < 0 || id >= L) continue;
    uint32_t pos = atomicAdd(&cursor[id / TJ1], 1u);
    if (pos < (uint64_t)nnz) bucket[pos] = ((uint32_t)b << 16) | (uint32_t)(id % TJ1);
  }
}

// zero-padded BF16 copy of X ([MB][D]) and, in FP8 mode, its E4M3-RNE cast for the forward MFMA
__global__ void k_prep_x(const uint16_t* __restrict__ X, int B, int D, int MB, uint16_t* __restrict__ Xb,
                         uint8_t* __restrict__ Xq) {
  const int64_t n = (int64_t)MB * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t v = (i / D) < B ? X[i] : 0u;
    Xb[i] = (uint16_t)v;
    if (Xq) Xq[i] = (uint8_t)f32_to_e4m3_rne_sat(bf16_to_f32(v));
  }
}

// dX[b][d] = sum over label ranges r (fixed order) of the FP32 partials
__global__ void k_dx_reduce(const float* __restrict__ part, int NR, int MB, int D, int B, float* __restrict__ dX) {
  const int64_t n = (int64_t)B * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int r = 0; r < NR; ++r) s += part[(int64_t)r * MB * D + i];
    dX[i] = s;
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
template <int MB, int WF, bool LOSS, bool ZOUT>
__global__ __launch_bounds__(256) void k_fwd_g(const uint8_t* __restrict__ W, const uint8_t* __restrict__ Xf,
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
  __shared__ __attribute__((aligned(16))) uint8_t smem[fwd_smem_bytes(MB)];
  __shared__ uint32_t ybits[TJ1 * (MB / 32)];    // positives, label-major: bit b & 31 of word [j][b >> 5]
  __shared__ float lred[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wb = wave / WJ, wj = wave % WJ;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tile = blockIdx.x;
  const int64_t tg = c0 / TJ1 + tile;          // global 128-label tile index
  const int jbase = tile * TJ1;                // first label of the tile, relative to c0
  const int64_t rowbytes = (int64_t)D * ESZ;

  for (int i = tid; i < TJ1 * (MB / 32); i += 256) ybits[i] = 0u;
  __syncthreads();
  {
    const uint64_t e0 = tile_off[tg];
    const uint64_t e1 = tile_off[tg + 1] < (uint64_t)bucket_cap ? tile_off[tg + 1] : (uint64_t)bucket_cap;
    for (uint64_t e = e0 + tid; e < e1; e += 256) {
      uint32_t v = bucket[e];
      uint32_t b = v >> 16, jl = v & (TJ1 - 1);
      if (b < (uint32_t)MB) atomicOr(&ybits[jl * (MB / 32) + (b >> 5)], 1u << (b & 31));
    }
  }

  f32x16_t acc[MI][NI];
  fwd_tile<MB, WF, RW, CW>(acc, smem, W + (c0 + jbase) * rowbytes, clen - jbase, Xf, rowbytes, tid, wb, wj);

  // epilogue: gradient straight from the accumulators. A lane holds one label and 4 groups of 4
  // consecutive samples of each 32 x 32 block; packing pairs to BF16 and swapping groups 1 <-> 0 and
  // 3 <-> 2 across the lane halves leaves 8 consecutive samples per lane and group pair, written
  // with one 16-byte store into the label-major chunk buffer G[label][sample].
  float lsum = 0.0f;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int jl = wj * CW + ni * 32 + l32;
      const bool jvalid = jbase + jl < clen;
      const int bb = wb * RW + mi * 32;
      const uint32_t yw = ybits[jl * (MB / 32) + (bb >> 5)];
      float gv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int bl = 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool valid = jvalid && (bb + bl < B);
        const bool y = (yw >> bl) & 1u;
        const float z = acc[mi][ni][i];
        gv[i] = valid ? bce_grad(z, y) : 0.0f;
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
      if constexpr (!ZOUT) {
        uint32_t pk[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pk[k] = pack_bf16x2(gv[2 * k], gv[2 * k + 1]);
        uint16_t* grow = G + (int64_t)(jbase + jl) * gpitch;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk[4 * u], pk[4 * u + 2], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk[4 * u + 1], pk[4 * u + 3], false, false);
          const i32x4_t out = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
          *(i32x4_t*)(grow + bb + 16 * u + 8 * hi) = out;
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

// Work-group: 2 * DS/32 waves (two per SIMD for DS = 128). Wave w works on the 32 features
// [dsl + 32 (w % ND), +32) of the slice; the two waves of a feature block split the other MFMA
// dimension (samples for dX, labels for dW) between them.
// Per 64-label tile t (double buffered in LDS, the next tile's loads in flight during this one):
//   G tile  [64][MB] BF16 (label-major, as the forward kernel writes it), fetched straight into LDS
//           with global_load_lds;
//   W tile  [64][DS] decoded to BF16 in LDS;
//   dX^T[d][b] += sum_j W^T[d][j] G^T[j][b]  (A = W^T and B = G^T, both by ds_read_b64_tr_b16)
//   dW^T[d][j]  = sum_b X^T[d][b] G[b][j]    (A = stationary X^T fragments in registers, B = G rows)
//   dW stays in the accumulators: one permlane32 swap gives every lane 2 x 8 consecutive features
//   of one label, which it updates with one Philox block each: t = fmaf(-lr, dW, w), hardware
//   stochastic rounding, one coalesced store per 8 weights. One barrier per tile.
template <int MB, int WF, int DS>
__global__ __launch_bounds__(DS * 4) void k_bwd_update(uint8_t* __restrict__ W, int D, int64_t c0, int clen,
                                                       const uint16_t* __restrict__ Xb,
                                                       const uint16_t* __restrict__ G,
                                                       float* __restrict__ part, int NR, int NS, float lr,
                                                       uint64_t seed, uint64_t step) {
  constexpr int ND = DS / 32;                  // feature blocks
  constexpr int NWV = 2 * ND, NT = 64 * NWV;   // waves, threads
  constexpr int ESZ = WF == W_BF16_ ? 2 : 1;
  constexpr int NB = MB / 32;
  constexpr bool SPLIT_B = NB >= 2;            // dX: the two waves split samples, else split K
  constexpr int NBW = SPLIT_B ? NB / 2 : NB;   // sample blocks per wave for dX
  constexpr int GTE = TJ2 * MB;                // G tile elements
  constexpr int GCM = MB / 8 - 1;              // G row: chunk mask
  constexpr int GRI = 512 / MB;                // G rows per 1 KiB global_load_lds instruction
  constexpr int WCPR = DS * ESZ / 16;          // 16-byte global W chunks per tile row
  constexpr int WPT = TJ2 * WCPR / NT;         // W chunks per thread
  static_assert(WPT >= 1 && TJ2 == 64, "tile split");
  __shared__ __attribute__((aligned(1024))) uint16_t Gs[2][GTE];
  __shared__ __attribute__((aligned(1024))) uint16_t Ws[2][TJ2 * DS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dblk = wave % ND, half = wave / ND;
  const int l32 = lane & 31, hi = lane >> 5, q = lane >> 4, li = lane & 15;
  // work-groups of one label range share its G tiles: keep them on one XCD (dispatch is round-robin)
  const int g = blockIdx.x, xcd = g & 7, kq = g >> 3;
  const int r = (kq / NS) * 8 + xcd, s = kq % NS;
  if (r >= NR) return;
  const int nt = (clen + TJ2 - 1) / TJ2;
  const int t0 = (int)((int64_t)nt * r / NR), t1 = (int)((int64_t)nt * (r + 1) / NR);
  const int dsl = s * DS;
  const int64_t rowbytes = (int64_t)D * ESZ;

  // stationary X^T fragments of this wave's 32 features: lane (d, 8 samples)
  s16x8_t xT[MB / 16];
  {
    const int d = dsl + dblk * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < MB / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) xT[kk][e] = (short)Xb[(kk * 16 + hi * 8 + e) * D + d];
  }
  f32x16_t accX[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) accX[nb] = f32x16_t{};

  // loop-invariant LDS element offsets
  //   dW operand B: G row j = half*32 + l32, chunk 2 kk + hi  = 2 (kk ^ gW1) + hW
  const int jW = half * 32 + l32;
  const int gW = row_swz<MB / 8>(jW);
  const int offW = jW * MB + 8 * (hi ^ (gW & 1));
  const int gW1 = gW >> 1;
  //   dX operands (transposing reads): rows jX and jX + 4 of each 16-label K step
  const int jX = 8 * (q >> 1) + (li >> 2);
  const int sA0 = row_swz<DS / 8>(jX), sA1 = row_swz<DS / 8>(jX + 4);
  const int sB0 = row_swz<MB / 8>(jX), sB1 = row_swz<MB / 8>(jX + 4);
  const int kx0 = SPLIT_B ? 0 : half * (TJ2 / 32);
  //     A = W^T: features dblk*32 + 16 (q&1) + 4 (li&3) .. +3
  const int cA = 4 * dblk + 2 * (q & 1) + ((li & 3) >> 1);
  const int offA0 = (16 * kx0 + jX) * DS + ((cA ^ sA0) << 3) + 4 * (li & 1);
  const int offA1 = (16 * kx0 + jX + 4) * DS + ((cA ^ sA1) << 3) + 4 * (li & 1);
  //     B = G^T: samples 32 blk + 16 (q&1) + 4 (li&3) .. +3 of sample block blk
  int offB0[NBW], offB1[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int blk = (SPLIT_B ? half * NBW : 0) + nb;
    const int cB = 4 * blk + 2 * (q & 1) + ((li & 3) >> 1);
    offB0[nb] = (16 * kx0 + jX) * MB + ((cB ^ sB0) << 3) + 4 * (li & 1);
    offB1[nb] = (16 * kx0 + jX + 4) * MB + ((cB ^ sB1) << 3) + 4 * (li & 1);
  }
  //   update: W row jW, chunks 4 dblk + 2u + hi
  const int sU = row_swz<DS / 8>(jW);
  const int offU0 = jW * DS + (((4 * dblk + hi) ^ sU) << 3);
  const int offU1 = jW * DS + (((4 * dblk + 2 + hi) ^ sU) << 3);

  auto load_g = [&](int t, int buf) {
    const uint16_t* gt = G + (int64_t)t * TJ2 * MB;
    for (int inst = wave; inst < MB / 8; inst += NWV) {
      const int row = inst * GRI + lane / (MB / 8), pos = lane & GCM;
      global_load_lds16(gt + row * MB + ((pos ^ row_swz<MB / 8>(row)) << 3), &Gs[buf][inst * 512]);
    }
  };
  i32x4_t wst[WPT];
  auto load_w = [&](int t) {
    const int jb = t * TJ2;
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int ci = tid + c * NT, jr = ci / WCPR, p = ci % WCPR;
      i32x4_t v = {0, 0, 0, 0};
      if (jb + jr < clen) v = *(const i32x4_t*)(W + (c0 + jb + jr) * rowbytes + (int64_t)dsl * ESZ + p * 16);
      wst[c] = v;
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int c = 0; c < WPT; ++c) {
      const int ci = tid + c * NT, jr = ci / WCPR, p = ci % WCPR;
      const int sw = row_swz<DS / 8>(jr);
      uint16_t* row = &Ws[buf][jr * DS];
      if constexpr (WF == W_BF16_) {
        *(i32x4_t*)(row + ((p ^ sw) << 3)) = wst[c];
      } else {
        i32x4_t lo, hi4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = (uint32_t)wst[c][w];
          const uint32_t p0 = e4m3_to_bf16(v & 0xff) | (e4m3_to_bf16((v >> 8) & 0xff) << 16);
          const uint32_t p1 = e4m3_to_bf16((v >> 16) & 0xff) | (e4m3_to_bf16(v >> 24) << 16);
          if (w < 2) { lo[2 * w] = (int)p0; lo[2 * w + 1] = (int)p1; }
          else { hi4[2 * (w - 2)] = (int)p0; hi4[2 * (w - 2) + 1] = (int)p1; }
        }
        *(i32x4_t*)(row + (((2 * p) ^ sw) << 3)) = lo;
        *(i32x4_t*)(row + (((2 * p + 1) ^ sw) << 3)) = hi4;
      }
    }
  };

  if (t0 < t1) {
    load_g(t0, 0);
    load_w(t0);
    store_w(0);
    __builtin_amdgcn_s_waitcnt(0);
  }
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    __syncthreads();                           // tile t resident; iteration t-1 fully done
    if (t + 1 < t1) { load_g(t + 1, buf ^ 1); load_w(t + 1); }
    const uint16_t* gs = Gs[buf];
    const uint16_t* ws = Ws[buf];

    // The two contractions, interleaved so that the independent dX MFMAs fill the dependency gaps
    // of the dW chain, with every LDS fragment read issued two steps ahead of its MFMA:
    //   dX^T[d][b] += W^T[d][j] G^T[j][b]    (M = d, N = b, K = j)   NDX MFMAs
    //   dW^T[d][j]  = X^T[d][b] G[b][j]      (M = d, N = j, K = b)   NDW MFMAs, one chain
    constexpr int NDW = MB / 16;
    constexpr int KXN = SPLIT_B ? TJ2 / 16 : TJ2 / 32;     // dX K steps of this wave
    constexpr int NDX = KXN * NBW;
    constexpr int NST = NDW > NDX ? NDW : NDX;
    constexpr int PF = 2;                                  // prefetch distance (steps)
    auto ldW = [&](int kk) { return *(const s16x8_t*)(gs + offW + 16 * (kk ^ gW1)); };
    auto ldXa = [&](int kx) {
      return join(lds_read_tr16(ws + offA0 + kx * 16 * DS), lds_read_tr16(ws + offA1 + kx * 16 * DS));
    };
    auto ldXb = [&](int x) {
      const int kx = x / NBW, nb = x % NBW;
      return join(lds_read_tr16(gs + offB0[nb] + kx * 16 * MB), lds_read_tr16(gs + offB1[nb] + kx * 16 * MB));
    };
    s16x8_t fW[NST + PF], fXa[KXN + 1], fXb[NST + PF];
    f32x16_t accW = f32x16_t{};
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (i < NDW) fW[i] = ldW(i);
      if (i < NDX) { if (i % NBW == 0) fXa[i / NBW] = ldXa(i / NBW); fXb[i] = ldXb(i); }
    }
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int p = i + PF;
      if (p < NDW) fW[p] = ldW(p);
      if (p < NDX) { if (p % NBW == 0) fXa[p / NBW] = ldXa(p / NBW); fXb[p] = ldXb(p); }
      if (i < NDW) accW = mfma_bf16(xT[i], fW[i], accW);
      if (i < NDX) accX[i % NBW] = mfma_bf16(fXa[i / NBW], fXb[i], accX[i % NBW]);
    }

    // the next tile's operands: wait for this thread's loads (issued a whole MFMA phase ago; the
    // previous tile's weight stores have had as long) and stage the W tile. The stores of this
    // tile's update then overlap the next tile's MFMAs instead of being waited for here.
    if (t + 1 < t1) {
      __builtin_amdgcn_s_waitcnt(0);
      store_w(buf ^ 1);
    }

    // fused SGD + stochastic rounding straight from the accumulators. Lane (l32, hi) holds label
    // half*32 + l32 and features 8 (i/4) + 4 hi + i%4; swapping register groups 1<->0 and 3<->2
    // across the two lane halves leaves features [16u + 8hi, +8) for u = 0, 1 in each lane.
    {
      const int jr = half * 32 + l32;
      const int jb = t * TJ2;
      const bool live = jb + jr < clen;
      const int64_t jg = c0 + jb + jr;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float dw[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (copy to scalars first: bit-casting an ext-vector element reference reads element 0)
          const float lo_v = accW[8 * u + e], hi_v = accW[8 * u + 4 + e];
          const auto sw = __builtin_amdgcn_permlane32_swap(f2u(lo_v), f2u(hi_v), false, false);
          dw[e] = __builtin_bit_cast(float, (uint32_t)sw[0]);
          dw[4 + e] = __builtin_bit_cast(float, (uint32_t)sw[1]);
        }
        const int dl = dblk * 32 + 16 * u + 8 * hi;            // feature offset within the slice
        const i32x4_t wv = *(const i32x4_t*)(ws + (u ? offU1 : offU0));
        const u32x4 rnd = rng_block(seed, step, ((uint64_t)jg * (uint64_t)D + (uint64_t)(dsl + dl)) >> 3);
        float tv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wb = (uint32_t)wv[e >> 1];
          const float w = u2f((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
          tv[e] = fmaf(-lr, dw[e], w);
        }
        uint8_t* dst = W + jg * rowbytes + (int64_t)(dsl + dl) * ESZ;
        if constexpr (WF == W_BF16_) {
          i32x4_t out;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = sr_bf16_into(0u, tv[2 * w], rng_pick_hi(rnd, 2 * w), false);
            out[w] = (int)sr_bf16_into(lo, tv[2 * w + 1], rng_pick_hi(rnd, 2 * w + 1), true);
          }
          if (live) *(i32x4_t*)dst = out;
        } else {
          uint32_t o0 = 0, o1 = 0;
          o0 = sr_e4m3_into<0>(o0, tv[0], rng_pick_hi(rnd, 0));
          o0 = sr_e4m3_into<1>(o0, tv[1], rng_pick_hi(rnd, 1));
          o0 = sr_e4m3_into<2>(o0, tv[2], rng_pick_hi(rnd, 2));
          o0 = sr_e4m3_into<3>(o0, tv[3], rng_pick_hi(rnd, 3));
          o1 = sr_e4m3_into<0>(o1, tv[4], rng_pick_hi(rnd, 4));
          o1 = sr_e4m3_into<1>(o1, tv[5], rng_pick_hi(rnd, 5));
          o1 = sr_e4m3_into<2>(o1, tv[6], rng_pick_hi(rnd, 6));
          o1 = sr_e4m3_into<3>(o1, tv[7], rng_pick_hi(rnd, 7));
          if (live) *(uint2*)dst = make_uint2(o0, o1);
        }
      }
    }
  }

  // this range's dX contribution, accumulated in place (fixed slot per range: deterministic).
  // With the K split (one sample block) the two waves of a feature block add in turn.
#pragma unroll
  for (int pass = 0; pass < (SPLIT_B ? 1 : 2); ++pass) {
    if (SPLIT_B || half == pass) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int b = (SPLIT_B ? half * NBW + nb : nb) * 32 + l32;
          const int d = dsl + dblk * 32 + 8 * ig + 4 * hi;
          f32x4_t* pp = (f32x4_t*)(part + ((int64_t)r * MB + b) * D + d);
          f32x4_t v = *pp;
          v[0] += accX[nb][4 * ig]; v[1] += accX[nb][4 * ig + 1];
          v[2] += accX[nb][4 * ig + 2]; v[3] += accX[nb][4 * ig + 3];
          *pp = v;
        }
    }
    if (!SPLIT_B && pass == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
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
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
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
  s.Cc = c;
  s.ntiles = (L + TJ1 - 1) / TJ1;
  // backward work-groups hold a whole CU (LDS) and those of one label range share an XCD: give
  // each of the 8 XCDs at most as many work-groups as it has CUs, so the launch is one round
  int64_t nt2 = (c + TJ2 - 1) / TJ2;
  int per_xcd = (device_cus() / 8) / s.NS;
  if (per_xcd < 1) per_xcd = 1;
  const int cap = 8 * per_xcd;
  s.NR = (int)(nt2 < cap ? nt2 : cap);
  size_t off = 0;
  const size_t A = 256;
  s.flags = off;    off = align_up(off + 64, A);
  s.tile_cnt = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.tile_off = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.bucket = off;   off = align_up(off + 4 * (size_t)(max_nnz > 0 ? max_nnz : 1), A);
  s.xb = off;       off = align_up(off + 2 * (size_t)s.MB * D, A);
  s.xq = off;       off = align_up(off + (wdtype == W_E4M3_ ? (size_t)s.MB * D : 0), A);
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
    const int grid2 = 8 * s.NS * ((NR + 7) / 8);
    kt_begin(KT_BWD, st, clen);
    if (s.DS == 128)
      hipLaunchKernelGGL((k_bwd_update<MB, WF, 128>), dim3(grid2), dim3(512), 0, st, W, a.D, c0, clen,
                         (const uint16_t*)(ws + s.xb), Gc, part, NR, s.NS, a.lr, a.seed, a.step);
    else
      hipLaunchKernelGGL((k_bwd_update<MB, WF, 64>), dim3(grid2), dim3(256), 0, st, W, a.D, c0, clen,
                         (const uint16_t*)(ws + s.xb), Gc, part, NR, s.NS, a.lr, a.seed, a.step);
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
    hipLaunchKernelGGL(k_fill_u32, dim3(1024), dim3(256), 0, st, (uint32_t*)(ws + s.part),
                       (int64_t)s.NR * s.MB * a.D, 0u);
    LAUNCH_CHECK();
  }
  if (a.B > 0 && a.row_ptr) {
    hipLaunchKernelGGL(k_label_count, dim3(a.B), dim3(64), 0, st, a.row_ptr, a.ids, a.B, a.nnz, a.L, cnt, flags);
    LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_label_scan, dim3(1), dim3(1024), 0, st, cnt, off, s.ntiles);
  LAUNCH_CHECK();
  if (a.B > 0 && a.row_ptr && a.nnz > 0) {
    hipLaunchKernelGGL(k_label_scatter, dim3(a.B), dim3(64), 0, st, a.row_ptr, a.ids, a.nnz, a.L, cnt,
                       (uint32_t*)(ws + s.bucket));
    LAUNCH_CHECK();
  }
  {
    const int64_t n = (int64_t)s.MB * a.D;
    const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_prep_x, dim3(blocks), dim3(256), 0, st, (const uint16_t*)a.X, a.B, a.D, s.MB,
                       (uint16_t*)(ws + s.xb), a.wdtype == W_E4M3_ ? ws + s.xq : (uint8_t*)nullptr);
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
    const int64_t n = (int64_t)a.B * a.D;
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
