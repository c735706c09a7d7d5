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
// Those two kernels and the chunk loop live in step_chunks.hip; this file holds the small kernels
// around them (label handling, X preparation, the dX and loss reductions), the workspace layout and
// the step's launch sequence.
#include "step_kernels.hpp"

#include <type_traits>
#include <vector>

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

// The prepared feature copies, zero-padded to MB samples, each element i of a copy taken from
// the sample b and feature k that position i holds:
//   Xb  BF16 X: row-major [MB][D], or (XLAY_XB) the BF16 stationary forward's A fragments: K step
//       kk (16 features) of wave w's 32 samples at ((w (D / 16) + kk) 64 + lane) 8, lane (l, h)
//       holding sample 32 w + l, features 16 kk + 8 h .. + 7;
//   Xq  (E4M3 and MXFP4 weights) E4M3-RNE(X): row-major, or (XLAY_XS_*) the stationary forward's A
//       fragments: 16-byte part p of K step kk (64 features) of wave w at (((w (D / 64) + kk) 2 +
//       p) 64 + lane) 16, lane (l, h) holding sample 32 w + l, features 64 kk + 32 h + 16 p .. + 15
//       (beside E4M3 weights) or 64 kk + 32 p + 16 h .. + 15 (beside E2M1 weights);
//   XbT BF16 X^T for the backward's stationary operand: feature block fb (32 features), sample
//       step kk (16 samples) at ((fb (MB / 16) + kk) 64 + lane) 8, lane (l, h) holding feature
//       32 fb + l, samples 16 kk + 8 h .. + 7.
// Every fragment load of the consuming kernels is then 1 KiB contiguous per wave.
__global__ void k_prep_x(const uint16_t* __restrict__ X, int B, int D, int MB, int xlay, uint16_t* __restrict__ Xb,
                         uint8_t* __restrict__ Xq, uint16_t* __restrict__ XbT) {
  const int64_t n = (int64_t)MB * D;
  auto at = [&](int64_t b, int64_t k) { return b < B ? (uint32_t)X[b * D + k] : 0u; };
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (xlay == XLAY_XB) {
      const int e = (int)(i & 7), lane = (int)((i >> 3) & 63);
      const int64_t r = i >> 9, kk = r % (D / 16), w = r / (D / 16);
      Xb[i] = (uint16_t)at(32 * w + (lane & 31), 16 * kk + 8 * (lane >> 5) + e);
    } else {
      Xb[i] = (uint16_t)at(i / D, i % D);
    }
    if (Xq) {
      int64_t b = i / D, k = i % D;
      if (xlay == XLAY_XS_E4M3 || xlay == XLAY_XS_MX) {
        const int e = (int)(i & 15), lane = (int)((i >> 4) & 63), part = (int)((i >> 10) & 1), h = lane >> 5;
        const int64_t r = i >> 11, kk = r % (D / 64), w = r / (D / 64);
        b = 32 * w + (lane & 31);
        k = 64 * kk + (xlay == XLAY_XS_MX ? 32 * part + 16 * h : 32 * h + 16 * part) + e;
      }
      Xq[i] = (uint8_t)f32_to_e4m3_rne_sat(bf16_to_f32(at(b, k)));
    }
    {
      const int e = (int)(i & 7), lane = (int)((i >> 3) & 63);
      const int64_t r = i >> 9, kk = r % (MB / 16), fb = r / (MB / 16);
      XbT[i] = (uint16_t)at(16 * kk + 8 * (lane >> 5) + e, 32 * fb + (lane & 31));
    }
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
  const int64_t rb = w_row_bytes(wdtype, D);
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
  // the single-pass step runs one work-group per CU over 32-label tiles, each with its own partial
  const int64_t nt1 = (c + 31) / 32;
  s.NR1 = single_pass_shape(s.MB, D) ? (int)(nt1 < s.cus ? nt1 : s.cus) : 0;
  const int nslots = s.NR > s.NR1 ? s.NR : s.NR1;
  size_t off = 0;
  const size_t A = 256;
  s.flags = off;    off = align_up(off + 64, A);
  s.tile_cnt = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.tile_off = off; off = align_up(off + 4 * (size_t)(s.ntiles + 1), A);
  s.bucket = off;   off = align_up(off + 4 * (size_t)(max_nnz > 0 ? max_nnz : 1), A);
  s.xb = off;       off = align_up(off + 2 * (size_t)s.MB * D, A);
  s.xq = off;       off = align_up(off + (wdtype != W_BF16_ ? (size_t)s.MB * D : 0), A);
  s.xbt = off;      off = align_up(off + 2 * (size_t)s.MB * D, A);
  s.g = off;        off = align_up(off + 2 * (size_t)s.MB * (size_t)s.Cc, A);
  s.part = off;     off = align_up(off + 4 * (size_t)nslots * s.MB * D, A);
  // loss partials: one slot per 128-, 64- or 32-label tile of the forward kernel in use
  s.loss = off;     off = align_up(off + 4 * (size_t)(4 * s.ntiles + 4), A);
  s.total = off;
  return s;
}

#define LAUNCH_CHECK() do { if (hipGetLastError() != hipSuccess) return ELMO_EHIP_; } while (0)


int run_step(const StepArgs& a, const StepLayout& s, void* workspace, hipStream_t st) {
  uint8_t* ws = (uint8_t*)workspace;
  uint32_t* flags = (uint32_t*)(ws + s.flags);
  uint32_t* cnt = (uint32_t*)(ws + s.tile_cnt);
  uint32_t* off = (uint32_t*)(ws + s.tile_off);
  // zero flags, tile counts and (for a training step) the dX partial sums
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, st, flags, (int64_t)16, 0u);
  hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(256), 0, st, cnt, s.ntiles + 1, 0u);
  LAUNCH_CHECK();
  if (a.loss) {
    // loss partials: one slot per 128-label tile (tiled forward) or per work-group and 64 or 32
    // labels (stationary-feature forwards); the slots a launch does not write stay zero
    hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(256), 0, st, (uint32_t*)(ws + s.loss), 4 * s.ntiles + 4, 0u);
    LAUNCH_CHECK();
  }
  if (!a.forward_only() && !a.single) {
    // the first chunk stores all partial slots unless it has fewer label ranges than there are slots
    // (the single-pass kernel always launches one work-group per slot)
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
                       fwd_x_layout(s.MB, a.wdtype, a.D), (uint16_t*)(ws + s.xb),
                       a.wdtype != W_BF16_ ? ws + s.xq : (uint8_t*)nullptr,
                       (uint16_t*)(ws + s.xbt));
    LAUNCH_CHECK();
  }
  int rc;
  const int MB = s.MB;
  if (a.single) {
    rc = a.wdtype == W_BF16_ ? run_single<W_BF16_>(a, s, ws, st)
       : a.wdtype == W_E4M3_ ? run_single<W_E4M3_>(a, s, ws, st) : run_single<W_MXFP4_>(a, s, ws, st);
  } else if (a.wdtype == W_BF16_) {
    rc = MB == 32 ? run_chunks<32, W_BF16_>(a, s, ws, st) : MB == 64 ? run_chunks<64, W_BF16_>(a, s, ws, st)
       : MB == 128 ? run_chunks<128, W_BF16_>(a, s, ws, st) : run_chunks<256, W_BF16_>(a, s, ws, st);
  } else if (a.wdtype == W_E4M3_) {
    rc = MB == 32 ? run_chunks<32, W_E4M3_>(a, s, ws, st) : MB == 64 ? run_chunks<64, W_E4M3_>(a, s, ws, st)
       : MB == 128 ? run_chunks<128, W_E4M3_>(a, s, ws, st) : run_chunks<256, W_E4M3_>(a, s, ws, st);
  } else {
    rc = MB == 32 ? run_chunks<32, W_MXFP4_>(a, s, ws, st) : MB == 64 ? run_chunks<64, W_MXFP4_>(a, s, ws, st)
       : MB == 128 ? run_chunks<128, W_MXFP4_>(a, s, ws, st) : run_chunks<256, W_MXFP4_>(a, s, ws, st);
  }
  if (rc != ELMO_OK_ || a.forward_only()) return rc;
  {
    const int64_t n = (int64_t)s.MB * a.D;
    const int blocks = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(k_dx_reduce, dim3(blocks), dim3(256), 0, st, (const float*)(ws + s.part), a.single ? s.NR1 : s.NR, s.MB,
                       a.D, a.B, a.dX);
    LAUNCH_CHECK();
  }
  if (a.loss) {
    hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(256), 0, st, (const float*)(ws + s.loss), 4 * s.ntiles + 4, a.loss);
    LAUNCH_CHECK();
  }
  return ELMO_OK_;
}

}  // namespace elmo