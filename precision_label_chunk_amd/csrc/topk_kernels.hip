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

TopkLayout topk_layout(int N, int D, int64_t L, int k, int wdtype) {
  TopkLayout s{};
  const int KK = k <= 8 ? 8 : k <= 32 ? 32 : 64;
  const int nbn = (N + TN - 1) / TN;
  s.MB = nbn * TN;                                    // padded sample count
  const int64_t ntile = (L + TJ1 - 1) / TJ1;
  int64_t want = (2 * (int64_t)device_cus() + nbn - 1) / nbn;
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

int run_topk(const void* W, int wdtype, int64_t L, int D, const void* X, int N, int k, int32_t* idx, float* score,
             const TopkLayout& s, void* workspace, hipStream_t st) {
  uint8_t* ws = (uint8_t*)workspace;
  const int64_t n = (int64_t)s.MB * D;
  const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
  hipLaunchKernelGGL(k_prep_eval_x, dim3(blocks), dim3(256), 0, st, (const uint16_t*)X, N, D, s.MB,
                     wdtype == W_BF16_ ? (uint16_t*)(ws + s.xb) : (uint16_t*)nullptr,
                     wdtype != W_BF16_ ? ws + s.xq : (uint8_t*)nullptr);
  if (hipGetLastError() != hipSuccess) return ELMO_EHIP_;
  if (k <= 8) return topk_launch<8>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
  if (k <= 32) return topk_launch<32>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
  return topk_launch<64>(W, wdtype, L, D, N, k, idx, score, s, ws, st);
}

}  // namespace elmo
