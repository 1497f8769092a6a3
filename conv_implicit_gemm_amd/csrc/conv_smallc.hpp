// conv_smallc.hpp -- implicit-GEMM convolution for inputs with few channels
// (C <= 4: the RGB stem of an image network), bf16, NCHW (instantiated by
// k_conv_smallc.hip).
//
// With C = 3 a reduction over channels alone cannot fill an MFMA's 16-deep
// k-step, so the k axis is ordered (kh, tap pair, channel) instead: the
// input band of a block is staged in LDS as 8-byte cells, one per input
// position, holding its (up to) 4 channels; a k-group of 8 values is then
// 2 horizontally adjacent taps x 4 channels, i.e. 2 adjacent cells of one
// patch row -- a single 16-byte LDS read for stride 2 (cell pairs start on
// an even column) and two 8-byte reads for stride 1.  One
// v_mfma_f32_32x32x16_bf16 step covers 4 taps of one kernel row (two
// k-groups); the kernel row's taps are padded to a multiple of 4 with zero
// weights, so a 7x7 kernel costs 7 x 2 steps (K = 224 for 147 real terms).
// The weights are rearranged into the same (kh, tap, channel) order while
// staged.  A block owns 64 output channels x TR output rows of one image;
// each of its four waves owns FP 32-pixel tiles x 64 channels.  The epilogue
// stages bf16 outputs in LDS as [channel][pixel] and writes channel runs
// with aligned vector stores.
#pragma once

#include "engine.hpp"

namespace ox {

namespace smallc {

constexpr int kCellB = 8;   // bytes per patch cell (4 bf16 channels)

template <int S, int NH, int FP, int P>
__global__ __launch_bounds__(kThreads, 2) void conv_smallc_bf16(const ConvArgs a, const SmallcPlan pl) {
  constexpr int FC = 2, BM = 64, WN = 4;
  constexpr int KROW = NH * 32;             // weight bytes per kernel row (4*NH taps x 4 ch x 2 B)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wn = tid >> 6;
  const int l32 = lane & 31, kg = lane >> 5;
  const int kH = a.kH, kW = a.kW, C = a.C, H = a.H, W = a.W, M = a.M;
  const int wrow = kH * KROW + 16;           // staged weight row (bytes), padded
  const int K = C * kH * kW;                  // weights per output channel
  char* As = smem;                            // weights [64][wrow]
  char* Ps = smem + BM * wrow;                // patch [PR][PWc] cells
  uint16_t* Wraw = (uint16_t*)(Ps + pl.PR * pl.PWc * kCellB);   // the block's weight rows as stored

  const int npb = pl.nrb * a.N;
  const int tile_id = xcd_tile(blockIdx.x, npb * pl.nmb);
  const int mb = tile_id / npb;
  const int rest = tile_id - mb * npb;
  const int n = rest / pl.nrb;
  const int oh0 = (rest - n * pl.nrb) * pl.TR;
  const int m0 = mb * BM;
  const int rows_here = min(pl.TR, a.Ho - oh0);
  const int ih_base = oh0 * S - a.pt;

  // Staging issues every global load before its first wait: the block's
  // weight rows (one contiguous range of mvalid*K values, 16-byte vectors
  // where W is aligned: WV per thread, a loop takes any rest), the input
  // band's 8-position groups (XV per thread; a group's rows outside the
  // image load row 0 or H-1 and are not stored).  The LDS tile is zeroed
  // while they are in flight.
  constexpr int WV = 6, XV = 2;
  const uint16_t* Wg = (const uint16_t*)a.Wt + (int64_t)m0 * K;
  const int wcount = min(BM, M - m0) * K;
  const int nvec = pl.w_vec ? wcount / 8 : 0;
  u32x4_t wv[WV];
  if (nvec > 0) {
#pragma unroll
    for (int k = 0; k < WV; ++k) wv[k] = *(const u32x4_t*)(Wg + min(tid + k * kThreads, nvec - 1) * 8);
  }
  const uint16_t* Xn = (const uint16_t*)a.X + (int64_t)n * C * H * W;
  const int ngrp = W / 8;
  const int nunits = P == 8 ? pl.PR * ngrp : 0;
  u32x4_t xv[XV][4];
  auto unit_src = [&](int u, int c) {        // channel c (clamped to C-1) of band group u
    const int pr = u / ngrp, j = u - (u / ngrp) * ngrp;
    const int ih = min(max(ih_base + pr, 0), H - 1);
    return Xn + ((int64_t)min(c, C - 1) * H + ih) * W + j * 8;
  };
  if (nunits > 0) {
#pragma unroll
    for (int k = 0; k < XV; ++k) {
      const int u = min(tid + k * kThreads, nunits - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[k][c] = *(const u32x4_t*)unit_src(u, c);
    }
  }
  // zero the patch and the weight tile (padding taps and channels stay 0)
  const int zbytes = BM * wrow + pl.PR * pl.PWc * kCellB;
  for (int i = tid * 16; i < zbytes; i += kThreads * 16) *(u32x4_t*)(smem + i) = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  // (the bias after the zeroing: its loads are waited for with the staging data)
  const uint16_t* bias = (const uint16_t*)a.bias;
  uint32_t braw[2];   // raw bits, converted in the epilogue (see the 3x3 kernel)
#pragma unroll
  for (int fc = 0; fc < 2; ++fc) {
    const int ml = fc * 32 + l32;
    braw[fc] = (bias && m0 + ml < M) ? (uint32_t)bias[m0 + ml] : 0u;
  }

  // weights, as stored, to Wraw (rearranged into (kh, tap, channel) order below)
  if (pl.w_vec) {
#pragma unroll
    for (int k = 0; k < WV; ++k)
      if (tid + k * kThreads < nvec) *(u32x4_t*)(Wraw + (tid + k * kThreads) * 8) = wv[k];
    for (int v = tid + WV * kThreads; v < nvec; v += kThreads)
      *(u32x4_t*)(Wraw + v * 8) = *(const u32x4_t*)(Wg + v * 8);
    for (int e = nvec * 8 + tid; e < wcount; e += kThreads) Wraw[e] = Wg[e];
  } else {
    for (int e = tid; e < wcount; e += kThreads) Wraw[e] = Wg[e];
  }
  // input band: patch cell (pr, pc) = input (ih_base + pr, pc - pl), channels 0..C-1
  if constexpr (P == 8) {
    auto put = [&](int u, const u32x4_t (&v)[4]) {
      const int pr = u / ngrp, j = u - (u / ngrp) * ngrp;
      const int ih = ih_base + pr;
      if (ih < 0 || ih >= H) return;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pc = j * 8 + e + a.pl;
        if (pc >= pl.PWc) break;
        const int sh = (e & 1) * 16, w = e >> 1;
        uint32_t cw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) cw[c] = c < C ? (v[c][w] >> sh) & 0xffffu : 0u;
        *(u32x2_t*)(Ps + (pr * pl.PWc + pc) * kCellB) = u32x2_t{cw[0] | (cw[1] << 16), cw[2] | (cw[3] << 16)};
      }
    };
#pragma unroll
    for (int k = 0; k < XV; ++k)
      if (tid + k * kThreads < nunits) put(tid + k * kThreads, xv[k]);
    for (int u = tid + XV * kThreads; u < nunits; u += kThreads) {
      u32x4_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = *(const u32x4_t*)unit_src(u, c);
      put(u, v);
    }
  } else {
    for (int u = tid; u < pl.PR * W; u += kThreads) {
      const int pr = u / W, iw = u - (u / W) * W;
      const int ih = ih_base + pr;
      const int pc = iw + a.pl;
      if (ih < 0 || ih >= H || pc >= pl.PWc) continue;
      uint32_t cv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) cv[c] = c < C ? Xn[((int64_t)c * H + ih) * W + iw] : 0u;
      *(u32x2_t*)(Ps + (pr * pl.PWc + pc) * kCellB) = u32x2_t{cv[0] | (cv[1] << 16), cv[2] | (cv[3] << 16)};
    }
  }
  __syncthreads();
  // rearrange: 16-byte piece (m, kh, j) holds taps 2j, 2j+1 x channels 0..3
  {
    const int mvalid = min(BM, M - m0);
    const int npc = 2 * NH;                   // pieces per kernel row
    for (int it = tid; it < mvalid * kH * npc; it += kThreads) {
      const int m = it / (kH * npc);
      const int r2 = it - m * (kH * npc);
      const int kh = r2 / npc, j = r2 - (r2 / npc) * npc;
      uint32_t d[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kw = 2 * j + t;
        uint32_t c4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          c4[c] = (kw < kW && c < C) ? Wraw[m * K + (c * kH + kh) * kW + kw] : 0u;
        d[2 * t] = c4[0] | (c4[1] << 16);
        d[2 * t + 1] = c4[2] | (c4[3] << 16);
      }
      *(u32x4_t*)(As + m * wrow + kh * KROW + j * 16) = u32x4_t{d[0], d[1], d[2], d[3]};
    }
  }
  __syncthreads();

  // this lane's pixel in each of the wave's FP tiles
  int pbase[FP];
#pragma unroll
  for (int f = 0; f < FP; ++f) {
    const int q = (wn * FP + f) * 32 + l32;
    const int r = q / a.Wo, ox = q - (q / a.Wo) * a.Wo;
    const bool valid = r < rows_here;
    pbase[f] = (valid ? (r * S) * pl.PWc + ox * S : 0) * kCellB + kg * 16;
  }
  const int wbase = l32 * wrow + kg * 16;

  f32x16_t acc[FP][FC];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FC; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // k-step (kh, h): pair kg of half h covers taps 4h + 2kg, 4h + 2kg + 1
  auto pix = [&](int off) -> u32x4_t {
    if constexpr (S == 2) {
      return *(const u32x4_t*)(Ps + off);
    } else {
      const u32x2_t lo = *(const u32x2_t*)(Ps + off), hi = *(const u32x2_t*)(Ps + off + 8);
      return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  for (int kh = 0; kh < kH; ++kh) {
    u32x4_t pf[NH][FP], wf[NH][FC];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
      for (int f = 0; f < FP; ++f) pf[h][f] = pix(pbase[f] + (kh * pl.PWc + 4 * h) * kCellB);
#pragma unroll
      for (int f = 0; f < FC; ++f) wf[h][f] = *(const u32x4_t*)(As + wbase + f * 32 * wrow + kh * KROW + h * 32);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int fp = 0; fp < FP; ++fp)
#pragma unroll
        for (int fc = 0; fc < FC; ++fc) mma32(acc[fp][fc], pf[h][fp], wf[h][fc]);
  }

  // epilogue: E[channel][pixel slot], then channel runs to Y
  __syncthreads();
  const int nslot = WN * FP * 32;
  const int erow = nslot + 8;
  uint16_t* E = (uint16_t*)smem;
  float bv[FC];
#pragma unroll
  for (int fc = 0; fc < FC; ++fc) bv[fc] = __uint_as_float(braw[fc] << 16);
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int fc = 0; fc < FC; ++fc) {
      const int ml = fc * 32 + l32;
#pragma unroll
      for (int fp = 0; fp < FP; ++fp) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int slot = (wn * FP + fp) * 32 + 8 * g + 4 * kg;
          const f32x16_t& c = acc[fp][fc];
          const uint32_t lo = pack_bf16x2(act_c<ACT>(c[4 * g + 0] + bv[fc]), act_c<ACT>(c[4 * g + 1] + bv[fc]));
          const uint32_t hi = pack_bf16x2(act_c<ACT>(c[4 * g + 2] + bv[fc]), act_c<ACT>(c[4 * g + 3] + bv[fc]));
          *(u32x2_t*)(E + ml * erow + slot) = u32x2_t{lo, hi};
        }
      }
    }
  });
  __syncthreads();
  uint16_t* Y = (uint16_t*)a.Y;
  const int HoWo = a.Ho * a.Wo;
  const int L = rows_here * a.Wo;
  const int g0 = oh0 * a.Wo;
  const int mvalid = min(BM, M - m0);
  int V = 8;
  while (V > 1 && ((HoWo % V) || (g0 % V) || (L % V) || (((uintptr_t)Y) % (2 * V)))) V >>= 1;
  const int per_run = L / V;
  for (int it = tid; it < mvalid * per_run; it += kThreads) {
    const int m = it / per_run;
    const int e = (it - m * per_run) * V;
    const uint16_t* src = E + m * erow + e;
    uint16_t* dst = Y + ((int64_t)n * M + m0 + m) * HoWo + g0 + e;
    if (V == 8) {
      const u32x2_t p0 = *(const u32x2_t*)src, p1 = *(const u32x2_t*)(src + 4);
      *(u32x4_t*)dst = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
    } else if (V == 4) {
      *(u32x2_t*)dst = *(const u32x2_t*)src;
    } else if (V == 2) {
      *(uint32_t*)dst = *(const uint32_t*)src;
    } else {
      *dst = *src;
    }
  }
}

}  // namespace smallc

}  // namespace ox
