// The forward contraction of one (all-samples x 128-label) tile on the matrix cores, shared by the
// training step's forward kernel and the top-k scoring kernel:
//   acc[b][j] = sum_k Xf[b][k] * W[j][k]
// with Xf the zero-padded feature rows (BF16, or E4M3 for E4M3 weights) and W the tile's weight
// rows (rows at or beyond `nvalid` read as zero). Operands are staged through LDS in K slices of
// KS bytes of every row (two LDS stages). Each slice's global loads are issued two slices ahead,
// spread over the MFMA slots of the slice before the one whose end writes them to LDS, so that
// neither a burst of loads stalls the wave at the memory queue nor the loads' latency sits
// between slices; MFMA operands are read from LDS one slot ahead of their use.
#pragma once
#include <type_traits>

#include "mfma.hpp"
#include "step_kernels.hpp"

namespace elmo {

constexpr int fwd_pitch(int KS) { return KS + 16; }     // LDS row pitch: conflict-free 16-row reads
constexpr int fwd_smem_bytes(int MB, int KS) { return 2 * (MB + TJ1) * fwd_pitch(KS); }

// RW x CW is this wave's sub-tile (RW samples, CW labels); the work-group is (MB/RW) x (TJ1/CW) waves
// SPREAD: the write-group row spreading below (off only where its few extra registers do not fit)
template <int MB, int WF, int RW, int CW, int KS, bool SPREAD = true, typename Mid>
__device__ __forceinline__ void fwd_tile(f32x16_t (&acc)[RW / 32][CW / 32], uint8_t* smem,
                                         const uint8_t* __restrict__ Wt, int nvalid,
                                         const uint8_t* __restrict__ Xf, int64_t rowbytes, int tid, int wb,
                                         int wj, Mid&& mid) {
  constexpr int MI = RW / 32, NI = CW / 32;
  constexpr int PT = fwd_pitch(KS);
  constexpr int SLICE = (MB + TJ1) * PT;
  constexpr int PPR = KS / 16;                           // 16-byte parts per row and slice
  constexpr int NCH = (MB + TJ1) * PPR;                  // chunks per slice
  constexpr int CPT = (NCH + 255) / 256;                 // chunks per thread
  constexpr int KSTEP = WF == W_BF16_ ? 32 : 64;         // K bytes per MFMA
  constexpr int NKK = KS / KSTEP;                        // MFMA K steps per slice
  constexpr int NSL = NKK * MI * NI;                     // MFMA slots per slice
  static_assert(KS % KSTEP == 0, "slice holds whole MFMA K steps");
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int nks = (int)((rowbytes + KS - 1) / KS);

  // chunk c of this thread: ci = tid + 256 c, part ci % PPR of a row (X rows, then W rows). The
  // 16 chunks of a ds_write_b128 lane group take rows PPR apart (4 rows of 64 bytes, or 2 of 128)
  // rather than consecutive ones: at the 80- or 144-byte pitch those land on disjoint bank windows,
  // where consecutive rows would overlap. Within each block of 16 rows, group m = (ci / 16) % PPR
  // holds rows m, m + PPR, ...; a chunk index past the last row maps past it as well.
  // Buffer loads: W rows at or past nvalid fall outside their resource and read as zero, and so
  // does a part past the end of a row (its offset is pushed out of range); whether chunk c is an X
  // or a W chunk is known at compile time when the X chunks fill whole multiples of 256.
  constexpr int NCHX = MB * PPR;                          // X chunks per slice
  constexpr int OOB = 0x7ffffff0;
  static_assert(MB % 16 == 0 && (PPR == 4 || PPR == 8), "whole 16-row blocks");
  auto chunk_row = [](int ci) {
    if constexpr (!SPREAD) return ci / PPR;
    const int g = ci >> 4;
    return 16 * (g / PPR) + g % PPR + PPR * ((ci & 15) / PPR);
  };
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(Xf, (int64_t)MB * rowbytes);
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(Wt, (int64_t)(nvalid < TJ1 ? nvalid : TJ1) * rowbytes);
  i32x4_t stg[2][CPT];
  auto gload = [&](auto S, auto K, int ks) {
    constexpr int c = decltype(K)::value;
    const int ci = tid + 256 * c, row = chunk_row(ci), part = ci % PPR;
    const int kb = ks * KS;                               // wave-uniform
    const bool inrow = kb + part * 16 < rowbytes;
    i32x4_t v = {0, 0, 0, 0};
    if constexpr (256 * (c + 1) <= NCHX) {
      v = buffer_load16(xres, inrow ? row * (int)rowbytes + part * 16 : OOB, kb);
    } else if constexpr (256 * c >= NCHX) {
      v = buffer_load16(wres, inrow ? (row - MB) * (int)rowbytes + part * 16 : OOB, kb);
    } else {
      const bool isx = row < MB;
      const i32x4_t vx = buffer_load16(xres, inrow && isx ? row * (int)rowbytes + part * 16 : OOB, kb);
      const i32x4_t vw = buffer_load16(wres, inrow && !isx ? (row - MB) * (int)rowbytes + part * 16 : OOB, kb);
      v = i32x4_t{vx[0] | vw[0], vx[1] | vw[1], vx[2] | vw[2], vx[3] | vw[3]};
    }
    stg[decltype(S)::value][c] = v;
  };
  auto lstore1 = [&](auto S, auto K, int buf) {
    constexpr int c = decltype(K)::value;
    const int ci = tid + 256 * c;
    if (c + 1 < CPT || ci < NCH)
      *(i32x4_t*)(smem + buf * SLICE + chunk_row(ci) * PT + (ci % PPR) * 16) = stg[decltype(S)::value][c];
  };
  auto lstore = [&](auto S, int buf) { static_for<0, CPT>([&](auto K) { lstore1(S, K, buf); }); };

  static_for<0, MI * NI>([&](auto I) { acc[decltype(I)::value / NI][decltype(I)::value % NI] = f32x16_t{}; });

  using Frag = typename std::conditional<WF == W_BF16_, s16x8_t, i32x8_t>::type;
  auto rdfrag = [&](const uint8_t* base, int row, int kk) -> Frag {
    const uint8_t* p = base + row * PT + kk * KSTEP + hi * (KSTEP / 2);
    if constexpr (WF == W_BF16_) {
      return *(const s16x8_t*)p;
    } else {
      const i32x4_t x0 = *(const i32x4_t*)p, x1 = *(const i32x4_t*)(p + 16);
      return i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  };

  // slice ks from LDS stage ks & 1 (parity S = ks & 1 at compile time): its MFMAs, with the loads of
  // slice ks + 2 (into staging set S) and the LDS writes of slice ks + 1 (staging set S ^ 1, loaded
  // during slice ks - 1, into the other stage, which every wave finished reading before the last
  // barrier) spread over its slots
  auto slice = [&](auto S, int ks) {
    constexpr int SP = decltype(S)::value;
    const uint8_t* Xs = smem + SP * SLICE;
    const uint8_t* Ws = Xs + MB * PT;
    Frag fa[NKK][MI], fb[NKK][NI];
    auto fetch = [&](auto Z) {                           // operands first used at slot Z + 1 (or Z = 0)
      constexpr int z = decltype(Z)::value;
      static_for<0, NKK * MI>([&](auto I) {
        constexpr int kk = decltype(I)::value / MI, mi = decltype(I)::value % MI;
        constexpr int f = (kk * MI + mi) * NI - 1;
        if constexpr ((f < 0 ? 0 : f) == z) fa[kk][mi] = rdfrag(Xs, wb * RW + mi * 32 + l32, kk);
      });
      static_for<0, NKK * NI>([&](auto I) {
        constexpr int kk = decltype(I)::value / NI, ni = decltype(I)::value % NI;
        constexpr int f = kk * MI * NI + ni - 1;
        if constexpr ((f < 0 ? 0 : f) == z) fb[kk][ni] = rdfrag(Ws, wj * CW + ni * 32 + l32, kk);
      });
    };
    static_for<0, NSL>([&](auto Z) {
      constexpr int z = decltype(Z)::value;
      constexpr int kk = z / (MI * NI), mi = (z / NI) % MI, ni = z % NI;
      fetch(Z);
      static_for<0, CPT>([&](auto K) {
        if constexpr (decltype(K)::value * NSL / CPT == z) {
          gload(S, K, ks + 2);
          if (ks + 1 < nks) lstore1(std::integral_constant<int, SP ^ 1>{}, K, SP ^ 1);
        }
      });
      if constexpr (WF == W_BF16_) acc[mi][ni] = mfma_bf16(fa[kk][mi], fb[kk][ni], acc[mi][ni]);
      else acc[mi][ni] = mfma_e4m3(fa[kk][mi], fb[kk][ni], acc[mi][ni]);
      sched_fence();
    });
    __syncthreads();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  static_for<0, CPT>([&](auto K) { gload(S0{}, K, 0); });
  static_for<0, CPT>([&](auto K) { gload(S1{}, K, 1); });
  mid();
  lstore(S0{}, 0);
  __syncthreads();
  for (int ks = 0; ks < nks; ks += 2) {
    slice(S0{}, ks);
    if (ks + 1 < nks) slice(S1{}, ks + 1);
  }
}

}  // namespace elmo
