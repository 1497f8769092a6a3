// conv_patch.hpp -- implicit-GEMM 3x3 convolution, bf16, with the input
// patch staged once per channel chunk (instantiated by k_conv_patch_*.hip).
//
// The generic implicit GEMM gathers every (channel, tap) element of its
// operand from global memory, i.e. each input value is fetched once per tap.
// Here a block owns BM = 32*WM*FC output channels and a band of TR output
// rows (or IMB whole images), and for each chunk of 32 input channels:
//   * stages the input band (with its halo, zero-filled once) in LDS in a
//     channel-contiguous layout: one 80-byte cell per input position holds
//     the 32 channels (64 bytes) plus 16 bytes of bank padding.  A staging
//     unit is P (1, 2, 4 or 8: the widest that keeps every plane's start
//     aligned) consecutive plane positions x 8 channels: 8 loads of P
//     elements, transposed by position (byte permutes) after the barrier.
//     Consecutive lanes take consecutive position groups, so global loads are
//     contiguous across a wave and the 16-byte cell writes hit distinct LDS
//     banks;
//   * stages the weights of the chunk tap-major.  ONNX-layout weights
//     W[m, c, kh, kw] are read as they lie in memory (8 channels x 9 taps =
//     9 aligned 16-byte loads) and permuted in registers so that each tap
//     holds its 32 channels contiguously; weights packed offline in that
//     tap-major order (ox_conv2d_pack_weights) are a straight, coalesced copy;
//   * runs 9 taps x 2 (16-channel halves) x FP x FC v_mfma_f32_32x32x16_bf16
//     per wave.  The pixel operand of output pixel p for tap (kh, kw) is the
//     cell at p's patch position plus a tap offset, so both MFMA fragments are
//     single 128-bit LDS reads.
// Each wave owns a (32*FP pixels) x (32*FC channels) tile: with FP = FC = 2 a
// 32x32x16 MFMA (full rate with only a few accumulators) consumes 1 KB of
// fragment reads per 32 cycles, which the LDS sustains for four waves.
// Columns of the patch are stored de-interleaved by stride phase (S = 2: all
// even columns, then all odd ones), so consecutive output pixels read
// consecutive cells for stride 2 as well as stride 1.
// The next chunk's global loads (raw-buffer loads, 2P bytes per channel
// and unit, branch-free) are interleaved with the first half of the current
// chunk's MFMAs and land in registers; one LDS buffer, two barriers per
// chunk.  The epilogue stores straight from the accumulators: each lane
// holds four consecutive output pixels of one channel.
#pragma once

#include <algorithm>

#include "engine.hpp"

namespace ox {

namespace patch {

constexpr int kCell = 80;     // bytes per patch cell
constexpr int kKK = 9;
constexpr int kAROW = kKK * 64 + 16;   // bytes per staged weight row

// staging registers of a unit (8 channels x P positions): one dword per
// channel up to P = 2, P/2 dwords per channel beyond
constexpr int patch_unit_dwords(int P) { return P <= 2 ? 8 : 4 * P; }
// staging units per thread: 64 (P = 1) or 32 staging registers, half that
// where the weight tile of a 128-channel block needs the room, at least one unit
constexpr int patch_upt(int P, int BM) {
  return (P == 1 ? 64 : 32) / (BM >= 128 ? 2 : 1) / patch_unit_dwords(P) > 0
             ? (P == 1 ? 64 : 32) / (BM >= 128 ? 2 : 1) / patch_unit_dwords(P)
             : 1;
}

// Geometry of logical tile `tile_id`: first output channel, first image,
// first output row, rows and images actually present.  The logical order
// cuts the (pixel block x channel block) grid into ga x gb equal rectangles,
// one per XCD (xcd_tile hands each XCD one contiguous eighth of the order),
// each walked channel block fastest: an XCD then re-reads its input bands
// (for its channel blocks) and its weight rows (for its pixel blocks) from
// its own L2.  ga = gb = 1: channel-block-major order.
struct TileGeo {
  int m0, img0, oh0, rows_here, imgs_here;
};
__device__ __forceinline__ TileGeo tile_geo(const ConvArgs& a, const PatchPlan& pp, int tile_id, int BM) {
  const int npb = pp.nrb * pp.nib;
  int mb, bx;
  if (pp.ga * pp.gb > 1) {
    const int rp = npb / pp.ga, rm = pp.nmb / pp.gb;   // exact: the planner checks
    const int r = div_small(tile_id, rp * rm), w = tile_id - r * (rp * rm);
    const int ri = div_small(r, pp.gb), rj = r - ri * pp.gb;
    const int wq = div_small(w, rm);
    bx = ri * rp + wq;
    mb = rj * rm + (w - wq * rm);
  } else {
    mb = div_small(tile_id, npb);
    bx = tile_id - mb * npb;
  }
  TileGeo t;
  const int ib = div_small(bx, pp.nrb);
  t.m0 = mb * BM;
  t.img0 = ib * pp.IMB;
  t.oh0 = (bx - ib * pp.nrb) * pp.TR;
  t.rows_here = min(pp.TR, a.Ho - t.oh0);
  t.imgs_here = min(pp.IMB, a.N - t.img0);
  return t;
}

// The direct-store epilogue: bias (fp32, from LDS),
// activation, bf16 rounding and stores of a wave's (32*FP pixel) x (32*FC
// channel) tile.
template <int FP, int FC>
__device__ __forceinline__ void store_acc(const ConvArgs& a, const PatchPlan& pp, const f32x16_t (&acc)[FP][FC],
                                          const float* Bs, int wm, int wn, int l32, int kg, int m0, int img0,
                                          int oh0, int rows_here, int imgs_here) {
  const int M = a.M;
  const int ppi = pp.TR * a.Wo;
  // Straight from the accumulators.  Lane (l32, kg) holds, for
  // each (fp, fc), output channel 32*fc + l32 at pixel slots 8*g + 4*kg +
  // (0..3), g = 0..3, of pixel tile fp: four consecutive slots of one
  // channel, which are four consecutive output pixels of one NCHW plane
  // whenever they lie in one image's band.  Bias, activation and bf16
  // rounding happen here; four such pixels at an 8-byte aligned address go
  // out as one store, any other slot element by element.  (The bias reads
  // LDS, published by the chunk loop's barriers.)
  uint16_t* Y = (uint16_t*)a.Y;
  const int HoWo = a.Ho * a.Wo;
  const int Lb = rows_here * a.Wo;             // output pixels of each image's band
  const int g0 = oh0 * a.Wo;                   // first of them in its plane
  float bv[FC];
#pragma unroll
  for (int fc = 0; fc < FC; ++fc) bv[fc] = Bs[wm * FC * 32 + fc * 32 + l32];
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int fp = 0; fp < FP; ++fp) {
      const int tile = wn * FP + fp;
      if (tile >= pp.NT) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int slot = tile * 32 + 8 * g + 4 * kg;
        const int i = div_small(slot, ppi);
        const int e = slot - i * ppi;           // position in image i's band
#pragma unroll
        for (int fc = 0; fc < FC; ++fc) {
          const int m = m0 + wm * FC * 32 + fc * 32 + l32;
          if (m >= M) continue;
          const f32x16_t& c = acc[fp][fc];
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = act_c<ACT>(c[4 * g + j] + bv[fc]);
          const int64_t off = ((int64_t)(img0 + i) * M + m) * HoWo + g0 + e;
          if (i < imgs_here && e + 3 < Lb && (off & 3) == 0) {
            *(u32x2_t*)(Y + off) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // (with several images per block the slots may reach further images)
              const int ij = div_small(slot + j, ppi), ej = slot + j - ij * ppi;
              if (ij < imgs_here && ej < Lb)
                Y[((int64_t)(img0 + ij) * M + m) * HoWo + g0 + ej] =
                    (uint16_t)(pack_bf16x2(v[j], 0.f) & 0xffffu);
            }
          }
        }
      }
    }
  });
}

template <int WM, int WN, int FP, int FC, int P, int S, bool WPACK>
__global__ __launch_bounds__(kThreads, (WM * FC * 32 == 64 ? 2 : 1)) void conv3x3_patch_bf16(
    const ConvArgs a, const PatchPlan pp) {
  constexpr int BM = 32 * WM * FC;          // output channels per block
  constexpr int UPT = patch_upt(P, BM);     // patch staging units per thread (max)
  constexpr int XC = patch_unit_dwords(P) / 8;   // staging dwords per channel of a unit
  // weight staging units per thread: packed layout, one 16-byte vector of a
  // channel row's 576 bytes each; ONNX layout, 8 channels x 9 taps each
  constexpr int WUNITS = WPACK ? BM * 36 / kThreads : BM * 4 / kThreads;
  constexpr int NLW = WUNITS * (WPACK ? 1 : kKK);   // weight loads per thread and chunk
  constexpr int NL = NLW + UPT * 8;                  // all loads per thread and chunk
  static_assert(WM * WN == 4, "four waves");
  static_assert(P == 1 || P == 2 || P == 4 || P == 8, "staging width");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* As = smem;
  char* Ps = smem + BM * kAROW;
  // the tile's fp32 bias, beyond the operand and epilogue areas: fetched with
  // the first chunk and written to LDS with it, so no wait lands early
  float* Bs = (float*)(smem + pp.lds - BM * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l32 = lane & 31, kg = lane >> 5;
  // logical unit: channel-block major, so that the blocks of one XCD share
  // their weight rows; with split-K a unit is one slice of a tile's
  // channel chunks, the slices of a tile adjacent
  const int tiles = pp.nrb * pp.nib * pp.nmb;
  const int unit = xcd_tile(blockIdx.x, tiles * pp.splits);
  const int tile_id = div_small(unit, pp.splits);
  const int slice = unit - tile_id * pp.splits;
  const TileGeo geo = tile_geo(a, pp, tile_id, BM);
  const int m0 = geo.m0, img0 = geo.img0, oh0 = geo.oh0;
  const int rows_here = geo.rows_here, imgs_here = geo.imgs_here;
  const int H = a.H, W = a.W, HW = H * W;
  const int C = a.C, M = a.M;
  const int K = C * kKK;
  const int ih_base = oh0 * a.sh - a.pt;
  const int ihs = max(0, ih_base), ihe = min(H, ih_base + pp.PR);
  const int flo = ihs * W, fhi = ihe * W;      // needed flat range of each plane
  const int fs = (flo / P) * P;
  const int ngrp = fhi > flo ? (fhi - fs + P - 1) / P : 0;
  const int units = imgs_here * 4 * ngrp;

  // Operands are read through raw buffers: a load whose offset lies past the
  // tensor returns zeros, so absent staging units, weight rows past M and the
  // loads after a slice's last chunk (offset with bit 31 set: every operand
  // is below 2^31 bytes) need no branch.
  constexpr uint32_t kPast = 0x80000000u;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.X), (short)0, (int)((uint32_t)a.N * (uint32_t)C * (uint32_t)HW * 2u), 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.Wt), (short)0, (int)((uint32_t)M * (uint32_t)K * 2u), 0x00020000);

  // staging units of this thread, fixed for every chunk: a unit is P
  // consecutive plane positions x 8 channels.  u_voff: byte offset of its
  // first value in the block's first chunk of channels (kPast: no unit);
  // u_lds: LDS byte offset of the cell of each position (-1: not needed).
  uint32_t u_voff[UPT];
  int u_lds[UPT][P];
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = tid + k * kThreads;
    u_voff[k] = kPast;
#pragma unroll
    for (int e = 0; e < P; ++e) u_lds[k][e] = -1;
    if (u < units) {
      const int i = div_small(u, 4 * ngrp);
      const int rem = u - i * 4 * ngrp;
      const int oct = div_small(rem, ngrp);
      const int g = rem - oct * ngrp;
      const int f0 = fs + g * P;
      u_voff[k] = (uint32_t)((((img0 + i) * C + oct * 8) * HW + f0) * 2);
      int ih = div_small(f0, W), iw = f0 - ih * W;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const int f = f0 + e;
        const int pc = iw + a.pl;
        if (f >= flo && f < fhi && pc < pp.PW) {
          const int cell =
              (i * pp.PR + ih - ih_base) * pp.PWt + (S == 1 ? pc : (pc & 1) * pp.PWs + (pc >> 1));
          u_lds[k][e] = cell * kCell + oct * 16;
        }
        if (++iw == W) {
          iw = 0;
          ++ih;
        }
      }
    }
  }
  // weight loads of this thread: byte offset of each in the block's first
  // chunk (kPast: row past M).  Packed: 16-byte vector j of row m's 576
  // bytes per chunk; ONNX layout: taps 0..8 of channel octet oct of row m.
  uint32_t w_voff[WUNITS];
#pragma unroll
  for (int k = 0; k < WUNITS; ++k) {
    const int v = tid + k * kThreads;
    if constexpr (WPACK) {
      const int m = v / 36, j = v - (v / 36) * 36;
      w_voff[k] = m0 + m < M ? (uint32_t)((m0 + m) * C * 18 + j * 16) : kPast;
    } else {
      const int m = v >> 2, oct = v & 3;
      w_voff[k] = m0 + m < M ? (uint32_t)((m0 + m) * K * 2 + oct * 144) : kPast;
    }
  }

  // this lane's pixel (row of the A operand) in each of the wave's FP tiles
  int pbase[FP];
  const int ppi = pp.TR * a.Wo;
#pragma unroll
  for (int f = 0; f < FP; ++f) {
    const int q = (wn * FP + f) * 32 + l32;
    const int i = div_small(q, ppi);
    const int rem = q - i * ppi;
    const int r = div_small(rem, a.Wo);
    const int c = rem - r * a.Wo;
    const bool valid = q < pp.NT * 32 && i < imgs_here && r < rows_here;
    pbase[f] = (valid ? (i * pp.PR + r * S) * pp.PWt + c : 0) * kCell + kg * 16;
  }
  int toff[kKK];
#pragma unroll
  for (int t = 0; t < kKK; ++t) {
    const int kh = t / 3, kw = t % 3;
    const int cw = kw * a.dw;
    toff[t] = (kh * a.dh * pp.PWt + (cw % S) * pp.PWs + cw / S) * kCell;
  }
  // this lane's weight row (column of the B operand) in each of FC tiles
  int wbase[FC];
#pragma unroll
  for (int f = 0; f < FC; ++f) wbase[f] = (wm * FC * 32 + f * 32 + l32) * kAROW + kg * 16;

  f32x16_t acc[FP][FC];
#pragma unroll
  for (int i = 0; i < FP; ++i)
#pragma unroll
    for (int j = 0; j < FC; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4_t wreg[WUNITS][WPACK ? 1 : kKK];
  uint32_t xv[UPT][8][XC];   // raw loaded values: per channel, P bf16 positions

  // load i (0 <= i < NL) of the chunk starting at channel c0; kill = kPast
  // sends it past the tensors (the slice has no further chunk)
  auto issue = [&](int i, int c0, uint32_t kill) {
    if (i < NLW) {
      const int k = WPACK ? i : i / kKK, j = WPACK ? 0 : i - (i / kKK) * kKK;
      wreg[k][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, (w_voff[k] | kill) + j * 16, c0 * 18, 0);
    } else {
      const int k = (i - NLW) >> 3, ch = (i - NLW) & 7;
      const uint32_t vo = u_voff[k] | kill;
      const int so = (c0 + ch) * HW * 2;
      if constexpr (P == 1) {
        xv[k][ch][0] = __builtin_amdgcn_raw_buffer_load_b16(xr, vo, so, 0);
      } else if constexpr (P == 2) {
        xv[k][ch][0] = __builtin_amdgcn_raw_buffer_load_b32(xr, vo, so, 0);
      } else if constexpr (P == 4) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(xr, vo, so, 0);
        xv[k][ch][0] = v[0];
        xv[k][ch][1] = v[1];
      } else {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, vo, so, 0);
        xv[k][ch][0] = v[0];
        xv[k][ch][1] = v[1];
        xv[k][ch][2] = v[2];
        xv[k][ch][3] = v[3];
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
          // the cell of position e: channels (2j, 2j+1) in dword j
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (P == 1) {
              d[j] = (xv[k][2 * j][0] & 0xffffu) | (xv[k][2 * j + 1][0] << 16);
            } else {
              const uint32_t lo = xv[k][2 * j][e >> 1], hi = xv[k][2 * j + 1][e >> 1];
              d[j] = __builtin_amdgcn_perm(hi, lo, (e & 1) ? 0x07060302u : 0x05040100u);
            }
          }
          *(u32x4_t*)(Ps + u_lds[k][e]) = u32x4_t{d[0], d[1], d[2], d[3]};
        }
      }
    }
  };

  const int nchunks = C / 32;
  const int c_lo = slice * pp.cps, c_hi = min(nchunks, c_lo + pp.cps);
#pragma unroll
  for (int i = 0; i < NL; ++i) issue(i, c_lo * 32, 0u);
  // while the first chunk is in flight: zero the whole patch once (halo
  // cells are never written again) and fetch this lane's bias values
  for (int i = tid; i < pp.npos * (kCell / 16); i += kThreads)
    *(u32x4_t*)(Ps + i * 16) = u32x4_t{0u, 0u, 0u, 0u};
  const uint16_t* bias = (const uint16_t*)a.bias;
  const uint32_t braw = (tid < BM && bias && m0 + tid < M) ? (uint32_t)bias[m0 + tid] : 0u;
  for (int chunk = c_lo; chunk < c_hi; ++chunk) {
    __syncthreads();                 // the previous chunk's MFMAs are done with LDS
    if (chunk == c_lo && tid < BM) Bs[tid] = __uint_as_float(braw << 16);
    store_chunk();
    __syncthreads();
    // The next chunk's loads are spread over the first half of this chunk's
    // k-steps, so that issuing them hides under matrix-core time (after the
    // slice's last chunk they are sent past the tensors: uniform code, no
    // branch).
    const int cn = (chunk + 1) * 32;
    const uint32_t kill = chunk + 1 < c_hi ? 0u : kPast;
    // 18 k-steps (9 taps x 2 halves of 16 channels).  Fragments are read two
    // steps ahead into a ring of three register sets, and the scheduler is
    // told to interleave those LDS reads and the loads one by one with the
    // MFMAs of the current step, so that their latency hides under
    // matrix-core time.
    constexpr int NS = 2 * kKK;
    u32x4_t pf[3][FP], wf[3][FC];
    auto read_frags = [&](int s, int buf) {
      const int t = s >> 1, h = (s & 1) * 32;
#pragma unroll
      for (int f = 0; f < FP; ++f) pf[buf][f] = *(const u32x4_t*)(Ps + pbase[f] + toff[t] + h);
#pragma unroll
      for (int f = 0; f < FC; ++f) wf[buf][f] = *(const u32x4_t*)(As + wbase[f] + t * 64 + h);
    };
    read_frags(0, 0);
    read_frags(1, 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool ahead = s + 2 < NS;
      if (ahead) read_frags(s + 2, (s + 2) % 3);
      // (over the first half of the steps, which leaves the second half's
      // matrix-core time for their latency)
      const int l0 = s < NS / 2 ? s * NL / (NS / 2) : NL, l1 = s < NS / 2 ? (s + 1) * NL / (NS / 2) : NL;
#pragma unroll
      for (int i = l0; i < l1; ++i) issue(i, cn, kill);
#pragma unroll
      for (int fp = 0; fp < FP; ++fp)
#pragma unroll
        for (int fc = 0; fc < FC; ++fc) mma32(acc[fp][fc], pf[s % 3][fp], wf[s % 3][fc]);
      constexpr int NM = FP * FC, NR = FP + FC;
      const int NV = l1 - l0;
#pragma unroll
      for (int i = 0; i < NM + NR + 8; ++i) {
        if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (ahead && i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global load
      }
      __builtin_amdgcn_sched_barrier(0);   // keep each step's reads in its own step
    }
  }

  if (pp.splits > 1) {
    // fp32 partial tile, [float4 index][thread] (coalesced for writer and reducer)
    f32x4_t* dst = (f32x4_t*)pp.ws + (int64_t)unit * (kThreads * FP * FC * 4) + tid;
#pragma unroll
    for (int fp = 0; fp < FP; ++fp)
#pragma unroll
      for (int fc = 0; fc < FC; ++fc)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dst[((fp * FC + fc) * 4 + g) * kThreads] =
              f32x4_t{acc[fp][fc][4 * g], acc[fp][fc][4 * g + 1], acc[fp][fc][4 * g + 2], acc[fp][fc][4 * g + 3]};
    return;
  }

  store_acc<FP, FC>(a, pp, acc, Bs, wm, wn, l32, kg, m0, img0, oh0, rows_here, imgs_here);
}

// Second pass of split-K: one block per (tile, wave of the first pass); its
// 256 threads split that wave's partial values four ways, add the slices in
// slice order, then bias, activation, bf16 and stores straight from the
// registers (four consecutive slots of one channel per value, as the first
// pass's direct epilogue writes them).
template <int WM, int WN, int FP, int FC>
__global__ __launch_bounds__(kThreads) void conv3x3_reduce(const ConvArgs a, const PatchPlan pp) {
  constexpr int BM = 32 * WM * FC;
  constexpr int SUBM = 32 * FC;
  constexpr int NV = FP * FC * 4, PER = NV / 4;
  // the first pass's order (xcd_tile over tile-major units): each XCD adds
  // the partials of the tiles its L2 wrote
  const int r = xcd_tile(blockIdx.x, gridDim.x);
  const int tile_id = r >> 2, w = r & 3;
  const int wm = w / WN, wn = w - (w / WN) * WN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, part = tid >> 6;
  const int l32 = lane & 31, kg = lane >> 5;
  const TileGeo geo = tile_geo(a, pp, tile_id, BM);
  const int M = a.M;
  // the bias of each value's channel, then every slice's partials
  float bvk[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int fc = ((part * PER + k) >> 2) % FC;
    bvk[k] = bias_bf16_at(a.bias, M, geo.m0 + wm * SUBM + fc * 32 + l32);
  }
  f32x4_t sum[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) sum[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  add_slices<PER>((const f32x4_t*)pp.ws + (int64_t)tile_id * pp.splits * (kThreads * NV) + w * 64 + lane +
                      part * PER * kThreads,
                  kThreads * NV, kThreads, pp.splits, sum);
  uint16_t* Y = (uint16_t*)a.Y;
  const int ppi = pp.TR * a.Wo, HoWo = a.Ho * a.Wo;
  const int Lb = geo.rows_here * a.Wo, g0 = geo.oh0 * a.Wo;
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = part * PER + k;             // value index (fp*FC + fc)*4 + g
      const int g = i & 3, fc = (i >> 2) % FC, fp = (i >> 2) / FC;
      const int tile = wn * FP + fp;
      const int m = geo.m0 + wm * SUBM + fc * 32 + l32;
      if (tile >= pp.NT || m >= M) continue;
      const int slot = tile * 32 + 8 * g + 4 * kg;
      const int ii = div_small(slot, ppi);
      const int e = slot - ii * ppi;            // position in image ii's band
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = act_c<ACT>(sum[k][j] + bvk[k]);
      const int64_t off = ((int64_t)(geo.img0 + ii) * M + m) * HoWo + g0 + e;
      if (ii < geo.imgs_here && e + 3 < Lb && (off & 3) == 0) {
        *(u32x2_t*)(Y + off) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ij = div_small(slot + j, ppi), ej = slot + j - ij * ppi;
          if (ij < geo.imgs_here && ej < Lb)
            Y[((int64_t)(geo.img0 + ij) * M + m) * HoWo + g0 + ej] = (uint16_t)(pack_bf16x2(v[j], 0.f) & 0xffffu);
        }
      }
    }
  });
}

template <int WM, int WN, int FP>
int launch_cfg(const ConvArgs& a, const PatchPlan& p, hipStream_t s) {
  constexpr int FC = 2;
  constexpr int BM = 32 * WM * FC;
  dim3 grid(p.nrb * p.nib * p.nmb * p.splits, 1, 1);
#define OX_PATCH_LAUNCH(P_, S_)                                                                  \
  do {                                                                                           \
    if (a.w_packed)                                                                              \
      hipLaunchKernelGGL((conv3x3_patch_bf16<WM, WN, FP, FC, P_, S_, true>), grid,               \
                         dim3(kThreads), p.lds, s, a, p);                                        \
    else                                                                                         \
      hipLaunchKernelGGL((conv3x3_patch_bf16<WM, WN, FP, FC, P_, S_, false>), grid,              \
                         dim3(kThreads), p.lds, s, a, p);                                        \
  } while (0)
  if (a.sw == 1) {
    if (p.VW == 8) OX_PATCH_LAUNCH(8, 1);
    else if (p.VW == 4) OX_PATCH_LAUNCH(4, 1);
    else if (p.VW == 2) OX_PATCH_LAUNCH(2, 1);
    else OX_PATCH_LAUNCH(1, 1);
  } else {
    if (p.VW == 8) OX_PATCH_LAUNCH(8, 2);
    else if (p.VW == 4) OX_PATCH_LAUNCH(4, 2);
    else if (p.VW == 2) OX_PATCH_LAUNCH(2, 2);
    else OX_PATCH_LAUNCH(1, 2);
  }
#undef OX_PATCH_LAUNCH
  if (p.splits > 1)
    hipLaunchKernelGGL((conv3x3_reduce<WM, WN, FP, FC>), dim3(p.nrb * p.nib * p.nmb * 4), dim3(kThreads),
                       0, s, a, p);
  return (int)hipGetLastError();
}

}  // namespace patch

// kernel configurations, one translation unit each: launch_patch_<WM>_<WN>_<FP>
// runs blocks of 64*WM output channels x 32*WN*FP pixel slots
int launch_patch_1_4_2(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_1_4_1(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_2_2_2(const ConvArgs& a, const PatchPlan& p, void* s);
int launch_patch_2_2_1(const ConvArgs& a, const PatchPlan& p, void* s);

}  // namespace ox
