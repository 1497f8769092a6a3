// conv_patch.hpp -- implicit-GEMM 3x3 convolution, bf16, with the input
// patch staged once per channel chunk (instantiated by k_conv_patch_*.hip).
//
// The generic implicit GEMM gathers every (channel, tap) element of its
// operand from global memory, i.e. each input value is fetched once per tap.
// Here a block owns BM output channels and a band of TR output rows (or IMB
// whole images) and, for each chunk of 32 input channels:
//   * stages the input band (with its halo, zero-filled once) in LDS in a
//     channel-contiguous layout: one 80-byte cell per input position holds the
//     32 channels (64 bytes) plus 16 bytes of bank padding.  A staging unit
//     is P (1 or 2) consecutive plane positions x 8 channels: 8 loads of P
//     elements, repacked by position in registers.  Consecutive lanes take
//     consecutive positions, so the global loads are contiguous across a wave
//     and the 16-byte cell writes hit distinct LDS banks;
//   * stages the weights of the chunk tap-major.  ONNX-layout weights
//     W[m, c, kh, kw] are read as they lie in memory (8 channels x 9 taps =
//     9 aligned 16-byte loads) and permuted in registers so that each tap
//     holds its 32 channels contiguously; weights packed offline in that
//     tap-major order (ox_conv2d_pack_weights) are a straight, coalesced copy;
//   * runs 9 taps x (BM/16) x (tiles of 16 pixels) MFMA 16x16x32 bf16: for tap
//     (kh, kw) the operand of output pixel p is the cell at p's patch position
//     plus a tap offset, so both MFMA fragments are single 128-bit LDS reads.
// Columns of the patch are stored de-interleaved by stride phase (S = 2: all
// even columns, then all odd ones), so consecutive output pixels read
// consecutive cells for stride 2 as well as stride 1.  Waves form a WM x
// (4/WM) grid over (output channels) x (pixel tiles).
// The next chunk's global loads are issued before the current chunk's MFMAs
// and land in registers; one LDS buffer, two barriers per chunk.
#pragma once

#include <algorithm>

#include "engine.hpp"

namespace ox {


namespace patch {

constexpr int kCell = 80;     // bytes per patch cell
// staging units per thread: 8 registers each, fewer where the accumulators
// of a wide wave tile need the room
constexpr int patch_upt(int P, int FN) { return (FN >= 4 ? 4 : 8) / P; }
constexpr int kKK = 9;
constexpr int kAROW = kKK * 64 + 16;

template <int BM, int WM, int FN, int P, int S, bool WPACK>
__global__ __launch_bounds__(kThreads, (BM == 64 ? 2 : 1)) void conv3x3_patch_bf16(const ConvArgs a,
                                                                                  const PatchPlan pp) {
  constexpr int WN = 4 / WM;                 // waves along the pixel tiles
  constexpr int FM = BM / (16 * WM);         // 16-row MFMA tiles per wave
  // weight staging units per thread: ONNX layout, 8 channels x 9 taps each;
  // packed layout, one 16-byte vector of a channel block's 576-byte row each
  constexpr int WUNITS = WPACK ? BM * 36 / kThreads : BM * 4 / kThreads;
  constexpr int UPT = patch_upt(P, FN);      // patch staging units per thread (max)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* As = smem;
  char* Ps = smem + BM * kAROW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int bx = blockIdx.x;
  const int img0 = (bx / pp.nrb) * pp.IMB;
  const int oh0 = (bx - (bx / pp.nrb) * pp.nrb) * pp.TR;
  const int rows_here = min(pp.TR, a.Ho - oh0);
  const int imgs_here = min(pp.IMB, a.N - img0);
  const int H = a.H, W = a.W, HW = H * W;
  const int C = a.C, M = a.M;
  const int K = C * kKK;
  const int ih_base = oh0 * a.sh - a.pt;
  const int ihs = max(0, ih_base), ihe = min(H, ih_base + pp.PR);
  const int flo = ihs * W, fhi = ihe * W;      // needed flat range of each plane
  const int fs = (flo / P) * P;
  const int ngrp = fhi > flo ? (fhi - fs + P - 1) / P : 0;
  const int units = imgs_here * 4 * ngrp;
  const uint16_t* Wt = (const uint16_t*)a.Wt;
  const uint16_t* Xblk = (const uint16_t*)a.X + (int64_t)img0 * C * HW;

  // zero the whole patch once: halo cells are never written again
  for (int i = tid; i < pp.npos * (kCell / 16); i += kThreads)
    *(u32x4_t*)(Ps + i * 16) = u32x4_t{0u, 0u, 0u, 0u};

  // staging units of this thread, fixed for every chunk: a unit is P
  // consecutive plane positions x 8 channels.  u_goff: element offset of its
  // first value from the chunk's first plane of image img0 (-1: no unit);
  // u_lds: LDS byte offset of the cell of each position (-1: not needed).
  int u_goff[UPT], u_lds[UPT][P];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = tid + k * kThreads;
    u_goff[k] = -1;
#pragma unroll
    for (int e = 0; e < P; ++e) u_lds[k][e] = -1;
    if (u < units) {
      const int i = u / (4 * ngrp);
      const int rem = u - i * 4 * ngrp;
      const int oct = rem / ngrp;
      const int g = rem - oct * ngrp;
      const int f0 = fs + g * P;
      u_goff[k] = (i * C + oct * 8) * HW + f0;
      int ih = f0 / W, iw = f0 - (f0 / W) * W;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const int f = f0 + e;
        const int pc = iw + a.pl;
        if (f >= flo && f < fhi && pc < pp.PW) {
          const int cell = (i * pp.PR + ih - ih_base) * pp.PWt + (S == 1 ? pc : (pc & 1) * pp.PWs + (pc >> 1));
          u_lds[k][e] = cell * kCell + oct * 16;
        }
        if (++iw == W) {
          iw = 0;
          ++ih;
        }
      }
    }
  }

  // this lane's output pixels (one per pixel tile the wave owns)
  int pbase[FN];
  bool pvalid[FN], pon[FN];
  int pimg[FN], prow[FN], pcol[FN];
  const int ppi = pp.TR * a.Wo;
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int j = wn + WN * f;
    const int q = j * 16 + lr;
    const int i = q / ppi;
    const int rem = q - i * ppi;
    const int r = rem / a.Wo;
    const int c = rem - r * a.Wo;
    pon[f] = j < pp.NT;
    pvalid[f] = pon[f] && i < imgs_here && r < rows_here;
    pimg[f] = i;
    prow[f] = r;
    pcol[f] = c;
    pbase[f] = pvalid[f] ? (i * pp.PR + r * S) * pp.PWt + c : 0;
  }
  int toff[kKK];
#pragma unroll
  for (int t = 0; t < kKK; ++t) {
    const int kh = t / 3, kw = t % 3;
    const int cw = kw * a.dw;
    toff[t] = kh * a.dh * pp.PWt + (cw % S) * pp.PWs + cw / S;
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t wreg[WUNITS][WPACK ? 1 : kKK];
  // raw loaded values (one per channel: P bf16 positions), repacked by
  // position only after the barrier so the loads stay in flight meanwhile
  uint32_t xreg[UPT][8];

  auto load_chunk = [&](int c0) {
    if constexpr (WPACK) {
      // packed: row m of chunk c0/32 is 9 taps x 32 channels, contiguous
#pragma unroll
      for (int k = 0; k < WUNITS; ++k) {
        const int v = tid + k * kThreads;
        const int m = v / 36, j = v - (v / 36) * 36;
        if (m0 + m < M)
          wreg[k][0] = *(const u32x4_t*)(Wt + ((int64_t)(m0 + m) * (C / 32) + c0 / 32) * 288 + j * 8);
        else
          wreg[k][0] = u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
#pragma unroll
      for (int k = 0; k < WUNITS; ++k) {
        const int u = tid + k * kThreads;
        const int m = u >> 2, oct = u & 3;
        if (m0 + m < M) {
          const uint16_t* src = Wt + (int64_t)(m0 + m) * K + (c0 + oct * 8) * kKK;
#pragma unroll
          for (int j = 0; j < kKK; ++j) wreg[k][j] = *(const u32x4_t*)(src + 8 * j);
        } else {
#pragma unroll
          for (int j = 0; j < kKK; ++j) wreg[k][j] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    const uint16_t* xc = Xblk + (int64_t)c0 * HW;
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      if (u_goff[k] >= 0) {
        const uint16_t* src = xc + u_goff[k];
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          if constexpr (P == 1) xreg[k][ch] = src[ch * HW];
          else xreg[k][ch] = *(const uint32_t*)(src + ch * HW);
        }
      }
    }
  };

  auto store_chunk = [&]() {
    if constexpr (WPACK) {
#pragma unroll
      for (int k = 0; k < WUNITS; ++k) {
        const int v = tid + k * kThreads;
        const int m = v / 36, j = v - (v / 36) * 36;
        *(u32x4_t*)(As + m * kAROW + j * 16) = wreg[k][0];
      }
    } else {
#pragma unroll
      for (int k = 0; k < WUNITS; ++k) {
        const int u = tid + k * kThreads;
        const int m = u >> 2, oct = u & 3;
        char* dst = As + m * kAROW + oct * 16;
#pragma unroll
        for (int t = 0; t < kKK; ++t) {
          // tap t of channels oct*8 .. oct*8+7: elements c*9 + t of the 72 loaded
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e0 = (2 * j) * kKK + t, e1 = (2 * j + 1) * kKK + t;
            const uint32_t w0 = wreg[k][e0 >> 3][(e0 & 7) >> 1];
            const uint32_t w1 = wreg[k][e1 >> 3][(e1 & 7) >> 1];
            const uint32_t lo = (e0 & 1) ? (w0 >> 16) : (w0 & 0xffffu);
            const uint32_t hi = (e1 & 1) ? (w1 & 0xffff0000u) : (w1 << 16);
            d[j] = lo | hi;
          }
          *(u32x4_t*)(dst + t * 64) = u32x4_t{d[0], d[1], d[2], d[3]};
        }
      }
    }
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
#pragma unroll
      for (int e = 0; e < P; ++e) {
        if (u_lds[k][e] >= 0) {
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = xreg[k][2 * j], hi = xreg[k][2 * j + 1];
            if constexpr (P == 1) d[j] = lo | (hi << 16);
            else if (e == 0) d[j] = (lo & 0xffffu) | (hi << 16);
            else d[j] = (lo >> 16) | (hi & 0xffff0000u);
          }
          *(u32x4_t*)(Ps + u_lds[k][e]) = u32x4_t{d[0], d[1], d[2], d[3]};
        }
      }
    }
  };

  const int nchunks = C / 32;
  load_chunk(0);
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    __syncthreads();                 // the previous chunk's MFMAs are done with LDS
    store_chunk();
    __syncthreads();
    if (chunk + 1 < nchunks) load_chunk((chunk + 1) * 32);
    // 9 taps; the fragments of tap t+1 are read while tap t's MFMAs run.
    // Every wave computes all FN tiles (a tile past NT reads cell 0 and is
    // discarded), which keeps the loop free of branches.
    u32x4_t af[2][FM], bf[2][FN];
    auto read_frags = [&](int t, int buf) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[buf][fm] = *(const u32x4_t*)(As + (wm * FM * 16 + fm * 16 + lr) * kAROW + t * 64 + lg * 16);
#pragma unroll
      for (int f = 0; f < FN; ++f)
        bf[buf][f] = *(const u32x4_t*)(Ps + (pbase[f] + toff[t]) * kCell + lg * 16);
    };
    read_frags(0, 0);
#pragma unroll
    for (int t = 0; t < kKK; ++t) {
      if (t + 1 < kKK) read_frags(t + 1, (t + 1) & 1);
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) Mma<DT_BF16>::run(acc[fm][f], bf[t & 1][f], af[t & 1][fm]);
    }
  }

  // Epilogue.  With the pixel operand first, lane (lr, lg) holds, for each
  // tile pair, output channel 16*fm + lr at the 4 consecutive pixel slots
  // 16*j + 4*lg .. +3.  Bias, activation and bf16 rounding happen here; the
  // block's tile is then staged in LDS as [channel][pixel slot] so that each
  // channel's run of output pixels (contiguous in NCHW) is written with the
  // widest aligned vector stores.
  __syncthreads();                       // all waves are done with the patch
  const int nslot = pp.NT * 16;
  const int erow = nslot + 8;            // elements per staged channel row
  uint16_t* E = (uint16_t*)smem;
  const uint16_t* bias = (const uint16_t*)a.bias;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int ml = wm * FM * 16 + fm * 16 + lr;
    const float bv = (bias && m0 + ml < M) ? bf16_to_f32(bias[m0 + ml]) : 0.0f;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int slot = (wn + WN * f) * 16 + lg * 4;
      if (slot < nslot) {
        uint32_t lo = (uint32_t)f32_to_bf16(apply_act(a.act, acc[fm][f][0] + bv)) |
                      ((uint32_t)f32_to_bf16(apply_act(a.act, acc[fm][f][1] + bv)) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(apply_act(a.act, acc[fm][f][2] + bv)) |
                      ((uint32_t)f32_to_bf16(apply_act(a.act, acc[fm][f][3] + bv)) << 16);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        *(u32x2_t*)(E + ml * erow + slot) = u32x2_t{lo, hi};
      }
    }
  }
  __syncthreads();
  // runs: for image i of the block and channel m, output pixels
  // [oh0*Wo, (oh0 + rows_here)*Wo) of plane (img0+i, m0+m) come from slots
  // [i*ppi, i*ppi + L)
  uint16_t* Y = (uint16_t*)a.Y;
  const int HoWo = a.Ho * a.Wo;
  const int L = rows_here * a.Wo;
  const int g0 = oh0 * a.Wo;
  const int mvalid = min(BM, M - m0);
  // widest vector that keeps every run's global and LDS start aligned
  int V = 8;
  while (V > 1 && ((HoWo % V) || (g0 % V) || (ppi % V) || (L % V) ||
                   (((uintptr_t)Y) % (2 * V))))
    V >>= 1;
  const int per_run = L / V;
  const int items = imgs_here * mvalid * per_run;
  for (int it = tid; it < items; it += kThreads) {
    const int run = it / per_run;
    const int e = (it - run * per_run) * V;
    const int i = run / mvalid;
    const int m = run - i * mvalid;
    const uint16_t* src = E + m * erow + i * ppi + e;
    uint16_t* dst = Y + ((int64_t)(img0 + i) * M + m0 + m) * HoWo + g0 + e;
    if (V == 8) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t p0 = *(const u32x2_t*)src, p1 = *(const u32x2_t*)(src + 4);
      *(u32x4_t*)dst = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
    } else if (V == 4) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      *(u32x2_t*)dst = *(const u32x2_t*)src;
    } else if (V == 2) {
      *(uint32_t*)dst = *(const uint32_t*)src;
    } else {
      *dst = *src;
    }
  }
}

template <int BM, int WM, int FN>
int launch_cfg(const ConvArgs& a, const PatchPlan& p, hipStream_t s) {
  dim3 grid(p.nrb * p.nib, (a.M + BM - 1) / BM, 1);
#define OX_PATCH_LAUNCH(P_, S_)                                                                   \
  do {                                                                                            \
    if (a.w_packed)                                                                               \
      hipLaunchKernelGGL((conv3x3_patch_bf16<BM, WM, FN, P_, S_, true>), grid, dim3(kThreads),  \
                         p.lds, s, a, p);                                                         \
    else                                                                                          \
      hipLaunchKernelGGL((conv3x3_patch_bf16<BM, WM, FN, P_, S_, false>), grid, dim3(kThreads), \
                         p.lds, s, a, p);                                                         \
  } while (0)
  if (a.sw == 1) {
    if (p.VW == 2) OX_PATCH_LAUNCH(2, 1);
    else OX_PATCH_LAUNCH(1, 1);
  } else {
    if (p.VW == 2) OX_PATCH_LAUNCH(2, 2);
    else OX_PATCH_LAUNCH(1, 2);
  }
#undef OX_PATCH_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace patch

// kernel configurations (one translation unit each)
int launch_patch_64_1_2(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_64_1_4(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_128_2_7(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_128_2_4(const ConvArgs& a, const PatchPlan& p, void* s);

}  // namespace ox
