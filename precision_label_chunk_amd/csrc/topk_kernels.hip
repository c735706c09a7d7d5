// Top-k label scoring for precision@k (ELMO summary page, "Experimental setup": P@1, P@3, P@5).
//
// score[n][j] = X~[n] . W[j] with the training forward's operands (X~ = E4M3-RNE(X) for E4M3
// weights), never materialised: each work-group owns 128 samples and one label range, computes
// 128 x 128 score tiles on the matrix cores (the same forward tile as the training step), stages
// each tile in LDS and lets two threads per sample keep running top-KK lists in registers (KK is k
// rounded up to 8, 32 or 64). Lists are ordered by (score desc, label asc) with NaN after numbers.
// Each list publishes its last entry's score in LDS as a bound: a tile's scores are first tested
// against the bounds in registers, and only those that may enter a list (usually none, once the
// lists have filled) go through an LDS queue to their list's thread; a tile with more such
// candidates than the queue holds takes the full path (the whole score tile through LDS).
// A second kernel merges the per-range lists of each sample.
#include <float.h>

#include "fwd_mx.hpp"
#include "fwd_tile.hpp"
#include "mfma.hpp"
#include "numerics.hpp"
#include "step_kernels.hpp"

namespace elmo {

constexpr int TN = 128;                 // samples per work-group
constexpr int QCAP = 256;               // candidate queue entries per tile

__device__ __forceinline__ bool ranks_before(float sa, int ja, float sb, int jb) {
  const bool na = sa != sa, nb = sb != sb;
  if (na != nb) return nb;
  if (!na && sa != sb) return sa > sb;
  return ja < jb;
}

template <int KK>
__device__ __forceinline__ void list_insert(float (&ls)[KK], int (&lj)[KK], float s, int j) {
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    if (ranks_before(s, j, ls[i], lj[i])) {
      const float ts = ls[i]; const int tj = lj[i];
      ls[i] = s; lj[i] = j; s = ts; j = tj;
    }
  }
}

template <int KK>
__device__ __forceinline__ void list_init(float (&ls)[KK], int (&lj)[KK]) {
#pragma unroll
  for (int i = 0; i < KK; ++i) { ls[i] = __builtin_nanf(""); lj[i] = INT32_MAX; }
}

// register i (dynamic) of a 16-register accumulator block, by a select chain
__device__ __forceinline__ float reg_pick16(const f32x16_t& a, int i) {
  float v = a[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) v = i == k ? a[k] : v;
  return v;
}

// (lists of 64 take the whole register file of a SIMD lane: one work-group per CU)
template <int WF, int KK>
__global__ __launch_bounds__(256, KK > 32 ? 1 : 2) void k_topk_scan(const uint8_t* __restrict__ W, int64_t L, int D,
                                                   const uint8_t* __restrict__ Xf, int nbn, int NRg,
                                                   float* __restrict__ cs, int* __restrict__ ci) {
  constexpr int MB = TN, RW = 64, CW = 64, MI = 2, NI = 2;
  constexpr int SP = TJ1 + 4;           // score tile pitch (floats)
  // K slice bytes (two work-groups per CU either way; 64 for E4M3 lists of 32, whose registers are
  // short for the larger staging)
  constexpr int KS = (WF == W_BF16_ || KK <= 8) ? 128 : 64;
  constexpr int SMEM = MB * SP * 4 > fwd_smem_bytes(MB, KS) ? MB * SP * 4 : fwd_smem_bytes(MB, KS);
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];   // operand stages, then the score tile
  // bound[h][n]: score of the last entry of sample n's list for label half h (NaN while not full)
  __shared__ __attribute__((aligned(16))) float bound[2][MB];
  __shared__ uint32_t qkey[QCAP];       // candidates: sample | half << 7 | label in tile << 8
  __shared__ float qscore[QCAP];
  __shared__ uint32_t qcount;
  __shared__ uint32_t wcand[4];         // per wave: it had candidates this tile

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wb = wave >> 1, wj = wave & 1, l32 = lane & 31, hi = lane >> 5;
  const int g = blockIdx.x, xcd = g & 7, kq = g >> 3;
  const int r = (kq / nbn) * 8 + xcd, nb = kq % nbn;   // one range's work-groups share an XCD
  if (r >= NRg) return;
  const int64_t ntile = (L + TJ1 - 1) / TJ1;
  const int64_t t0 = ntile * r / NRg, t1 = ntile * (r + 1) / NRg;
  const int64_t rowbytes = w_row_bytes(WF, D);
  // the block's feature rows: BF16 codes, or E4M3 codes for E4M3 and MXFP4 weights
  const uint8_t* Xblk = Xf + (int64_t)nb * MB * D * (WF == W_BF16_ ? 2 : 1);

  float ls[KK]; int lj[KK];
  list_init<KK>(ls, lj);
  const int srow = tid >> 1, half = tid & 1;
  float* sc = (float*)smem;
  bound[half][srow] = __builtin_nanf("");
  if (tid == 0) qcount = 0u;            // (the first tile's barriers order these before use)

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t j0 = t * TJ1;
    const int nvalid = (int)((L - j0) < TJ1 ? (L - j0) : TJ1);
    f32x16_t acc[MI][NI];
    if constexpr (WF == W_MXFP4_) {
      // (the tile's operands come straight from memory: the LDS staging area only holds scores)
      __syncthreads();                  // the previous tile's score reads are done
      mx_logit_tile<MI, NI>(acc, buffer_rsrc(Xblk, MB * D), wb * RW, D,
                            buffer_rsrc(W + j0 * rowbytes, nvalid * (int)rowbytes), wj * CW, (int)rowbytes, l32, hi);
    } else {
      fwd_tile<MB, WF, RW, CW, KS, KK <= 8>(acc, smem, W + j0 * rowbytes, nvalid, Xblk, rowbytes, tid, wb, wj, [] {});
    }

    if constexpr (KK <= 8) {
      // candidates: a score may enter its list only if the list's bound is NaN or not above it
      // (a bound from an earlier tile is a lower one, so it never drops a candidate); NaN scores
      // pass the test too and are sorted out by the list. Wave (wb, wj) holds samples
      // wb * RW .. + RW - 1 and label half wj (CW = 64) of the tile.
      uint32_t cm[MI * NI];               // candidate bits, register i of block (mi, ni)
      int cnt = 0;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int nb = wb * RW + mi * 32 + 4 * hi;
        f32x4_t bq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bq[q] = *(const f32x4_t*)&bound[wj][nb + 8 * q];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const bool jin = wj * CW + ni * 32 + l32 < nvalid;
          uint32_t m = 0u;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float b = bq[i >> 2][i & 3], z = acc[mi][ni][i];
            m |= (uint32_t)(jin && !(z < b)) << i;     // (also true when b or z is NaN)
          }
          cm[mi * NI + ni] = m;
          cnt += __builtin_popcount(m);
        }
      }
      // a wave with candidates queues them; only when the queue overflows do such waves write
      // their scores to the score tile, for the full path
      const bool wany = __builtin_amdgcn_ballot_w64(cnt > 0) != 0;
      if (wany) {
        // the lane's candidates into the queue (as far as it goes), each score taken from the
        // accumulators by a select over the block's 16 registers
        uint32_t k = cnt > 0 ? atomicAdd(&qcount, (uint32_t)cnt) : 0u;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            uint32_t m = cm[mi * NI + ni];
            while (m != 0u) {
              const int i = __builtin_ctz(m);
              m &= m - 1u;
              if (k < (uint32_t)QCAP) {
                const int n = wb * RW + mi * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
                qkey[k] = (uint32_t)n | ((uint32_t)wj << 7) | ((uint32_t)(wj * CW + ni * 32 + l32) << 8);
                qscore[k] = reg_pick16(acc[mi][ni], i);
              }
              ++k;
            }
          }
      }
      if (lane == 0) wcand[wave] = wany ? 1u : 0u;
      __syncthreads();
      const uint32_t nq = qcount;
      if (nq > (uint32_t)QCAP) {
        // too many for the queue: the waves with candidates write their scores to the tile
        if (wany) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                sc[(wb * RW + mi * 32 + 8 * (i >> 2) + 4 * hi + (i & 3)) * SP + wj * CW + ni * 32 + l32] = acc[mi][ni][i];
        }
        __syncthreads();
      }
      if (nq <= (uint32_t)QCAP) {
        // few candidates: each list's thread takes its own from the queue
        const uint32_t key = (uint32_t)srow | ((uint32_t)half << 7);
#pragma unroll 4
        for (uint32_t e = 0; e < nq; ++e) {
          const uint32_t v = qkey[e];
          if ((v & 0xffu) == key) {
            const float s = qscore[e];
            const int j = (int)(j0 + (v >> 8));
            if (ranks_before(s, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, s, j);
          }
        }
      } else if (wcand[(srow / RW) * 2 + half]) {
        // the row half from the score tile (written by the one wave that holds it)
        const int jend = nvalid < (half + 1) * 64 ? nvalid : (half + 1) * 64;
        for (int jl = half * 64; jl < jend; ++jl) {
          const float s = sc[srow * SP + jl];
          const int j = (int)(j0 + jl);
          if (ranks_before(s, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, s, j);
        }
      }
    } else {
      // (longer lists: registers are short for the candidate test; always the full path)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sc[(wb * RW + mi * 32 + 8 * (i >> 2) + 4 * hi + (i & 3)) * SP + wj * CW + ni * 32 + l32] = acc[mi][ni][i];
      __syncthreads();
      const int jend = nvalid < (half + 1) * 64 ? nvalid : (half + 1) * 64;
      for (int jl = half * 64; jl < jend; ++jl) {
        const float s = sc[srow * SP + jl];
        const int j = (int)(j0 + jl);
        if (ranks_before(s, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, s, j);
      }
    }
    bound[half][srow] = ls[KK - 1];
    __syncthreads();                    // scores and queue consumed before the next tile's staging
    if (tid == 0) qcount = 0u;
  }

  // merge the two half lists of each sample through LDS, then write this range's candidates
  float* ms = (float*)smem;
  int* mj = (int*)(smem + MB * KK * 4);
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < KK; ++i) { ms[srow * KK + i] = ls[i]; mj[srow * KK + i] = lj[i]; }
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      const float s = ms[srow * KK + i]; const int j = mj[srow * KK + i];
      if (ranks_before(s, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, s, j);
    }
    const int64_t base = ((int64_t)r * nbn * MB + (int64_t)nb * MB + srow) * KK;
#pragma unroll
    for (int i = 0; i < KK; ++i) { cs[base + i] = ls[i]; ci[base + i] = lj[i]; }
  }
}

// ------------------------------------------------------------------------------------------------
// top-k with the queries stationary in registers (MXFP4 weights, D = 768, lists of up to 8; the
// kernel also takes E4M3 weights)
// ------------------------------------------------------------------------------------------------
// The training forward's stationary layout (k_fwd_xs) applied to scoring: a work-group holds 256
// queries' E4M3 fragments in registers (wave w: queries 32 w .. 32 w + 31) and streams one label
// range's weights through LDS in 64-label tiles, three buffers deep, the two groups of four waves
// in complementary phases (the MFMAs of one overlapping the candidate pass of the other). The two
// lists of a query (label halves of each tile) live in the lanes of the wave that computes its
// scores: lane 2 m + h owns query 32 w + m, half h. The candidate pass is therefore wave-local: a
// score is a candidate only if it does not rank below its list's last entry (the lists' bounds in
// the wave's LDS region; a bound from an earlier tile is a lower one, so no entry is lost, and NaN
// bounds and scores pass); candidates go through the wave's LDS queue in rounds of QW entries (the
// first tiles of a range, where the lists fill, take several rounds), and no work-group barrier
// is needed beyond the tile pipeline's one per iteration. Work-group (range r, query block qb):
// the query blocks of one range run on one XCD (dispatch is round-robin over the 8 XCDs), so a
// range's weight tiles come from HBM about once per XCD and from L2 for the other blocks.
constexpr int TQ = 256;                 // queries per work-group of the stationary scan
constexpr int QW = 128;                 // wave queue entries per round

template <int WF>
__global__ __launch_bounds__(512, 1) void k_topk_xs(const uint8_t* __restrict__ W, int64_t L,
                                                  const uint8_t* __restrict__ Xq, int nbq, int NRg,
                                                  float* __restrict__ cs, int* __restrict__ ci) {
  constexpr int KK = 8;
  constexpr bool MX = WF == W_MXFP4_;
  constexpr int NK = 12, D_ = 64 * NK;
  constexpr int TJ = 64;                              // labels per tile
  constexpr int RB = MX ? D_ / 2 + D_ / 32 : D_;     // bytes per weight row
  constexpr int PITCH = MX ? 432 : D_ + 16;           // as in k_fwd_xs
  constexpr int PPR = D_ / 16;
  constexpr int NCH = MX ? TJ * RB / 16 : TJ * PPR;   // 16-byte chunks per tile
  constexpr int CPT = (NCH + 511) / 512;
  __shared__ __attribute__((aligned(16))) uint8_t Ws[3][TJ * PITCH];
  __shared__ __attribute__((aligned(16))) float bnd[8][2][32];   // per wave: bound of (half, query)
  __shared__ uint32_t qk[8][QW];                                  // per wave: owner lane | label << 6
  __shared__ float qs[8][QW];
  __shared__ uint32_t qn[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int l32 = lane & 31, hi = lane >> 5;
  const int bb = 32 * wave;
  const int g = blockIdx.x, xcd = g & 7, kq = g >> 3;
  const int r = (kq / nbq) * 8 + xcd, qb = kq % nbq;
  if (r >= NRg) return;
  const int64_t ntile = (L + TJ - 1) / TJ;
  const int t0 = (int)(ntile * r / NRg), t1 = (int)(ntile * (r + 1) / NRg);
  const int nmy = t1 - t0;
  const int64_t jbase = (int64_t)t0 * TJ;
  const int64_t rows = L - jbase < (int64_t)nmy * TJ ? L - jbase : (int64_t)nmy * TJ;
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + jbase * RB, (int)(rows * RB));
  constexpr int OOB = 0x7ffffff0;

  i32x4_t stg[CPT];
  auto wload = [&](int t, i32x4_t (&st)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int cix = tid + 512 * c;
      if constexpr (MX) {
        st[c] = buffer_load16(wres, cix < NCH ? t * TJ * RB + cix * 16 : OOB);
      } else {
        const int row = cix / PPR, part = cix % PPR;
        st[c] = buffer_load16(wres, row < TJ ? (t * TJ + row) * D_ + part * 16 : OOB);
      }
    }
  };
  auto wstore = [&](int buf, const i32x4_t (&st)[CPT]) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int cix = tid + 512 * c;
      if constexpr (MX) {
        if (cix < NCH) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int b = cix * 16 + 8 * h, row = b / RB, off = b - row * RB;
            *(i32x2_t*)(&Ws[buf][row * PITCH + off]) = i32x2_t{st[c][2 * h], st[c][2 * h + 1]};
          }
        }
      } else {
        const int row = cix / PPR, part = cix % PPR;
        if (row < TJ) *(i32x4_t*)(&Ws[buf][row * PITCH + part * 16]) = st[c];
      }
    }
  };

  // prologue: tiles 0 and 1, then the query fragments, all in flight together; the tiles' LDS
  // writes wait only for the tile loads (issued first)
  i32x8_t xf[NK];
  i32x4_t stg1[CPT];
  wload(0, stg);
  wload(1, stg1);
  {
    const uint8_t* xr = Xq + (int64_t)(qb * TQ + bb + l32) * D_ + (MX ? hi * 16 : hi * 32);
    constexpr int O2 = MX ? 32 : 16;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const i32x4_t a0 = *(const i32x4_t*)(xr + kk * 64), a1 = *(const i32x4_t*)(xr + kk * 64 + O2);
      xf[kk] = i32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    }
  }
  wstore(0, stg);
  wstore(1, stg1);
  float ls[KK]; int lj[KK];
  list_init<KK>(ls, lj);
  const int qo = lane >> 1, half = lane & 1;          // the list this lane owns
  bnd[wave][half][qo] = __builtin_nanf("");
  if (lane == 0) qn[wave] = 0u;
  __syncthreads();

  f32x16_t acc[2];
  auto mfmas = [&](int buf) {
    acc[0] = f32x16_t{}; acc[1] = f32x16_t{};
    if constexpr (MX) {
      const uint8_t* wb = &Ws[buf][l32 * PITCH + hi * 16];
      uint32_t scl[2][NK / 4];
      const uint32_t psel = hi ? 0x07050301u : 0x06040200u;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const uint8_t* sp = wb - hi * 16 + ni * 32 * PITCH + D_ / 2;
#pragma unroll
        for (int m = 0; m < NK / 4; ++m) {
          const i32x2_t rr = *(const i32x2_t*)(sp + 8 * m);
          scl[ni][m] = __builtin_amdgcn_perm((uint32_t)rr[1], (uint32_t)rr[0], psel);
        }
      }
      auto rd = [&](int z) { return *(const i32x4_t*)(wb + (z & 1) * 32 * PITCH + (z >> 1) * 32); };
      i32x4_t f[3];
      f[0] = rd(0); f[1] = rd(1);
      static_for<0, 2 * NK>([&](auto Z) {
        constexpr int z = decltype(Z)::value, kk = z >> 1;
        if constexpr (z + 2 < 2 * NK) f[(z + 2) % 3] = rd(z + 2);
        acc[z & 1] = mfma_e4m3_fp4_sel<kk % 4>(xf[kk], f[z % 3], acc[z & 1], (int)scl[z & 1][kk / 4]);
        sched_fence();
      });
    } else {
      const uint8_t* wb = &Ws[buf][l32 * PITCH + hi * 32];
      auto rd = [&](int z) {
        const uint8_t* p = wb + (z & 1) * 32 * PITCH + (z >> 1) * 64;
        const i32x4_t b0 = *(const i32x4_t*)p, b1 = *(const i32x4_t*)(p + 16);
        return i32x8_t{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      };
      i32x8_t f[3];
      f[0] = rd(0); f[1] = rd(1);
      static_for<0, 2 * NK>([&](auto Z) {
        constexpr int z = decltype(Z)::value;
        if constexpr (z + 2 < 2 * NK) f[(z + 2) % 3] = rd(z + 2);
        acc[z & 1] = mfma_e4m3(xf[z >> 1], f[z % 3], acc[z & 1]);
        sched_fence();
      });
    }
  };
  // the candidate pass of tile t of the range (wave-local)
  auto cand = [&](int t) {
    const int64_t j0 = jbase + (int64_t)t * TJ;
    uint32_t cm[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      // register i of block ni: query 8 (i >> 2) + 4 hi + (i & 3) of the wave, label ni * 32 + l32
      const float* bp = &bnd[wave][ni][4 * hi];
      f32x4_t b4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) b4[q] = *(const f32x4_t*)(bp + 8 * q);
      const bool jin = j0 + ni * 32 + l32 < L;
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) m |= (uint32_t)(jin && !(acc[ni][i] < b4[i >> 2][i & 3])) << i;
      cm[ni] = m;
    }
    if (__builtin_amdgcn_ballot_w64((cm[0] | cm[1]) != 0u) == 0) return;
    while (true) {
      const int cnt = __builtin_popcount(cm[0]) + __builtin_popcount(cm[1]);
      if (__builtin_amdgcn_ballot_w64(cnt > 0) == 0) break;
      uint32_t k = cnt > 0 ? atomicAdd(&qn[wave], (uint32_t)cnt) : 0u;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        uint32_t m = cm[ni], keep = 0u;
        while (m != 0u) {
          const int i = __builtin_ctz(m);
          m &= m - 1u;
          if (k < (uint32_t)QW) {
            const uint32_t q = 8u * (uint32_t)(i >> 2) + 4u * (uint32_t)hi + (uint32_t)(i & 3);
            qk[wave][k] = (2u * q + (uint32_t)ni) | ((uint32_t)(ni * 32 + l32) << 6);
            qs[wave][k] = reg_pick16(acc[ni], i);
          } else {
            keep |= 1u << i;
          }
          ++k;
        }
        cm[ni] = keep;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const uint32_t nq0 = qn[wave];
      const uint32_t nq = nq0 < (uint32_t)QW ? nq0 : (uint32_t)QW;
      for (uint32_t e = 0; e < nq; ++e) {
        const uint32_t v = qk[wave][e];
        if ((int)(v & 63u) == lane) {
          const float sc = qs[wave][e];
          const int j = (int)(j0 + (v >> 6));
          if (ranks_before(sc, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, sc, j);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane == 0) qn[wave] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    bnd[wave][half][qo] = ls[KK - 1];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  for (int i = 0; i <= nmy; ++i) {
    if (i + 2 < nmy) wload(i + 2, stg);
    const int ie = i - grp;                           // the tile whose candidates this wave passes
    if (grp == 0 && i < nmy) mfmas(i % 3);
    if (ie >= 0 && ie < nmy) cand(ie);
    if (grp == 1 && i < nmy) mfmas(i % 3);
    if (i + 2 < nmy) wstore((i + 2) % 3, stg);
    __syncthreads();
  }

  // merge each query's two half lists (lane pair), then write the range's candidates
#pragma unroll
  for (int i = 0; i < KK; ++i) {
    const float sc = __shfl_xor(ls[i], 1);
    const int j = __shfl_xor(lj[i], 1);
    if (half == 0 && ranks_before(sc, j, ls[KK - 1], lj[KK - 1])) list_insert<KK>(ls, lj, sc, j);
  }
  if (half == 0) {
    const int64_t base = ((int64_t)r * nbq * TQ + (int64_t)qb * TQ + bb + qo) * KK;
#pragma unroll
    for (int i = 0; i < KK; ++i) { cs[base + i] = ls[i]; ci[base + i] = lj[i]; }
  }
}

template <int KK>
__global__ __launch_bounds__(128) void k_topk_merge(const float* __restrict__ cs, const int* __restrict__ ci, int N, int Npad, int NRg,
                             int k, int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float ls[KK]; int lj[KK];
  list_init<KK>(ls, lj);
  for (int r = 0; r < NRg; ++r) {
    const int64_t base = ((int64_t)r * Npad + n) * KK;
    for (int i = 0; i < KK; ++i) {
      const float s = cs[base + i]; const int j = ci[base + i];
      if (!ranks_before(s, j, ls[KK - 1], lj[KK - 1])) break;   // per-range lists are sorted
      list_insert<KK>(ls, lj, s, j);
    }
  }
#pragma unroll
  for (int i = 0; i < KK; ++i)
    if (i < k) {
      out_idx[(int64_t)n * k + i] = lj[i];
      if (out_score) out_score[(int64_t)n * k + i] = ls[i];
    }
}

__global__ void k_prep_eval_x(const uint16_t* __restrict__ X, int N, int D, int Npad, uint16_t* __restrict__ Xb,
                              uint8_t* __restrict__ Xq) {
  const int64_t n = (int64_t)Npad * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t v = (i / D) < N ? X[i] : 0u;
    if (Xb) Xb[i] = (uint16_t)v;
    if (Xq) Xq[i] = (uint8_t)f32_to_e4m3_rne_sat(bf16_to_f32(v));
  }
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// the stationary-query scan serves MXFP4 weights at D = 768 with lists of up to 8 (top-5 of 4,096
// queries over 3M labels: 18.3 ms against 30 ms for the tiled scan, whose MX tile reads its
// operands from memory; for E4M3 the tiled scan, with its LDS-staged tile, stays faster: 16.5
// against 18.6 ms)
static bool topk_stationary(int D, int k, int wdtype) { return wdtype == W_MXFP4_ && D == 768 && k <= 8; }

TopkLayout topk_layout(int N, int D, int64_t L, int k, int wdtype) {
  TopkLayout s{};
  const int KK = k <= 8 ? 8 : k <= 32 ? 32 : 64;
  const bool xs = topk_stationary(D, k, wdtype);
  const int tn = xs ? TQ : TN;
  const int nbn = (N + tn - 1) / tn;
  s.MB = nbn * tn;                                    // padded sample count
  // label ranges: two work-groups per CU for the tiled scan, one for the stationary one (which
  // holds a whole CU's LDS), each range at least one tile
  const int64_t ntile = xs ? (L + 63) / 64 : (L + TJ1 - 1) / TJ1;
  const int64_t wgs = (xs ? 1 : 2) * (int64_t)device_cus();
  int64_t want = (wgs + nbn - 1) / nbn;
  // (the stationary scan addresses a range's weight rows through one buffer resource: at most
  // 1 GiB per range)
  if (xs) {
    const int64_t bytes = ntile * 64 * w_row_bytes(wdtype, D);
    const int64_t minr = (bytes + (int64_t(1) << 30) - 1) >> 30;
    if (want < minr) want = minr;
  }
  if (want < 1) want = 1;
  s.NRg = (int)(want < ntile ? want : ntile);
  s.ncand = (int64_t)s.NRg * s.MB * KK;
  size_t off = 0;
  s.xb = off; off = align256(off + (wdtype == W_BF16_ ? 2 * (size_t)s.MB * D : 0));
  s.xq = off; off = align256(off + (wdtype != W_BF16_ ? (size_t)s.MB * D : 0));
  s.cand_s = off; off = align256(off + 4 * (size_t)s.ncand);
  s.cand_i = off; off = align256(off + 4 * (size_t)s.ncand);
  s.total = off;
  return s;
}

template <int KK>
static int topk_launch(const void* W, int wdtype, int64_t L, int D, int N, int k, int32_t* idx, float* score,
                       const TopkLayout& s, uint8_t* ws, hipStream_t st) {
  const int nbn = s.MB / TN;
  const int grid = 8 * nbn * ((s.NRg + 7) / 8);
  float* cs = (float*)(ws + s.cand_s);
  int* ci = (int*)(ws + s.cand_i);
  if (wdtype == W_BF16_)
    hipLaunchKernelGGL((k_topk_scan<W_BF16_, KK>), dim3(grid), dim3(256), 0, st, (const uint8_t*)W, L, D,
                       (const uint8_t*)(ws + s.xb), nbn, s.NRg, cs, ci);
  else if (wdtype == W_E4M3_)
    hipLaunchKernelGGL((k_topk_scan<W_E4M3_, KK>), dim3(grid), dim3(256), 0, st, (const uint8_t*)W, L, D,
                       (const uint8_t*)(ws + s.xq), nbn, s.NRg, cs, ci);
  else
    hipLaunchKernelGGL((k_topk_scan<W_MXFP4_, KK>), dim3(grid), dim3(256), 0, st, (const uint8_t*)W, L, D,
                       (const uint8_t*)(ws + s.xq), nbn, s.NRg, cs, ci);
  if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  hipLaunchKernelGGL((k_topk_merge<KK>), dim3((N + 127) / 128), dim3(128), 0, st, cs, ci, N, s.MB, s.NRg, k, idx,
                     score);
  return hipGetLastError() == hipSuccess ? ELMO_OK_ : ELMO_EHIP_;
}

static int topk_launch_xs(const void* W, int wdtype, int64_t L, int N, int k, int32_t* idx, float* score,
                          const TopkLayout& s, uint8_t* ws, hipStream_t st) {
  const int nbq = s.MB / TQ;
  const int grid = 8 * nbq * ((s.NRg + 7) / 8);
  float* cs = (float*)(ws + s.cand_s);
  int* ci = (int*)(ws + s.cand_i);
  (void)wdtype;
  hipLaunchKernelGGL((k_topk_xs<W_MXFP4_>), dim3(grid), dim3(512), 0, st, (const uint8_t*)W, L,
                     (const uint8_t*)(ws + s.xq), nbq, s.NRg, cs, ci);
  if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  hipLaunchKernelGGL((k_topk_merge<8>), dim3((N + 127) / 128), dim3(128), 0, st, cs, ci, N, s.MB, s.NRg, k, idx,
                     score);
  return hipGetLastError() == hipSuccess ? ELMO_OK_ : ELMO_EHIP_;
}

int run_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k, int32_t* idx, float* score,
             const TopkLayout& s, void* workspace, hipStream_t st) {
  uint8_t* ws = (uint8_t*)workspace;
  const int64_t n = (int64_t)s.MB * D;
  const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
  hipLaunchKernelGGL(k_prep_eval_x, dim3(blocks), dim3(256), 0, st, (const uint16_t*)X, N, D, s.MB,
                     wdtype == W_BF16_ ? (uint16_t*)(ws + s.xb) : (uint16_t*)nullptr,
                     wdtype != W_BF16_ ? ws + s.xq : (uint8_t*)nullptr);
  if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  if (topk_stationary(D, k, wdtype)) return topk_launch_xs(W, wdtype, L, N, k, idx, score, s, ws, st);
  if (k <= 8) return topk_launch<8>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
  if (k <= 32) return topk_launch<32>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
  return topk_launch<64>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
}

}  // namespace elmo
