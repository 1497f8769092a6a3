// conv_pwd.hpp -- pointwise (1x1, stride 1, unpadded) bf16 convolution on
// NCHW with operands staged by DMA (instantiated by k_conv_pwd.hip).
//
// Y[n, m, p] = act(bias[m] + sum_c W[m, c] * X[n, c, p] (+ R[n, m, p])) is a
// GEMM over the flattened pixels of the batch, q = n*HW + p (the 1x1 fast
// path: a GEMM straight on the input, with no im2col).  The pixel tile is
// gathered in pieces of PB bytes (PB = 16: 8 pixels, when HW % 8 == 0; PB =
// 4: 2 pixels, when HW is even), each lane fetching its own piece, so that a
// piece never straddles two images and a tile may span images.
//
// Work split.  The grid is persistent: block (r, mb) owns output channels
// [mb*BC, mb*BC + BC) over pixel range r, one of nranges equal contiguous
// ranges of the batch's pixels (the last one shorter), each a whole number
// of 64- or 128-pixel units, so that row segments stay line-aligned and
// every block moves the same number of bytes (the slowest block sets the
// time; one tile per block would leave a tail of partly filled rounds).  A
// block walks its range in tiles of BP pixels.
//
// Pipeline.  The reduction over C runs in stages of KC channels through a
// ring of S LDS slots; each stage holds
//   * the KC x BP pixel tile as the image stores it (one row of BP
//     consecutive pixels per channel), and
//   * the BC x KC weight tile as W stores it (one row of KC channels per
//     output channel),
// both filled by buffer-to-LDS DMA (lds_dma.hpp) S-1 stages ahead of the
// MFMAs.  The block's stages form one stream across its tiles: the next
// tile's first stages are in flight while the current tile finishes and
// writes its outputs, and no staging register holds data in flight.
//
// Fragments: the pixel tile is the A operand of v_mfma_f32_32x32x16_bf16
// (rows = pixels), read with two ds_read_b64_tr_b16 per fragment straight
// from the channel rows; the weights are the B operand (columns = output
// channels), one 128-bit read per fragment.
//
// Epilogue: the tile goes through LDS as bf16 channel rows and each row
// segment is written by consecutive lanes (whole lines per instruction).
// With a residual it is written from the accumulators: lane l holds 4
// consecutive pixels of channel l%32 per accumulator group, lanes l and
// l+32 the two halves of an 8-pixel run, and one v_permlane32_swap per dword
// gives each lane a whole run of 8 pixels, read from R and written as 16
// bytes.
//
// Swizzles (16-byte pieces, applied by choosing which global piece each DMA
// lane fetches, and undone by the fragment addresses):
//   pixel rows of 256 B (BP = 128): piece j of channel row r sits at
//     j ^ ((r & 3) << 2) -- the 4 rows one half-wave reads through the
//     transposed read fall on 4 distinct 64-byte bank groups;
//   pixel rows of 128 B (BP = 64): j ^ (((r >> 1) & 1) << 2);
//   weight rows of 128 B (KC = 64): j ^ ((r >> 1) & 7), of 64 B (KC = 32):
//     j ^ ((r >> 2) & 3) -- the 16 rows of a quarter-wave's 128-bit reads
//     fall on distinct banks.
#pragma once

#include "lds_dma.hpp"

namespace ox {

namespace pwd {

template <int BP>
__device__ __forceinline__ int swz_x(int r) {
  if constexpr (BP == 128) return (r & 3) << 2;
  else return ((r >> 1) & 1) << 2;
}

template <int KC>
__device__ __forceinline__ int swz_w(int r) {
  if constexpr (KC == 64) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}

// Lanes l < 32 get (a[l], a[l+32]), lanes l >= 32 get (b[l-32], b[l]).
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

template <int BP, int BC, int KC, int S, int WP, int PB, bool RES>
__global__ __launch_bounds__(kThreads, 2) void conv1x1_dma(const ConvArgs a, const PwdPlan pl) {
  constexpr int WC = 4 / WP;
  constexpr int TP = BP / WP, TC = BC / WC;   // wave tile: pixels x channels
  constexpr int FP = TP / 32, FC = TC / 32;   // 32x32 fragments per wave
  constexpr int XROW = BP * 2;                // bytes per staged channel row of pixels
  constexpr int XB = KC * XROW;               // pixel tile bytes per stage
  constexpr int WROW = KC * 2;                // bytes per staged weight row
  constexpr int WB = BC * WROW;               // weight tile bytes per stage
  constexpr int SB = XB + WB;                 // stage bytes
  constexpr int XI = 64 * PB;                 // bytes of one pixel DMA instruction
  constexpr int IX = XB / (4 * XI), IW = WB / 4096;   // DMA instructions per wave per stage
  constexpr int D = IX + IW;
  constexpr int XPR = BP / 8, WPR = KC / 8;   // 16-byte pieces per row
  constexpr int SUB = 16 / PB;                // DMA pieces per 16-byte piece
  constexpr int NS = KC / 16;                 // k-steps per stage
  static_assert(WP * WC == 4 && FP >= 1 && FC >= 1, "four waves");
  static_assert(XB % (4 * XI) == 0 && WB % 4096 == 0, "whole DMA instructions per wave");
  static_assert(PB == 16 || PB == 4, "pixel DMA piece");
  static_assert(!RES || PB == 16, "the residual epilogue takes 8-pixel runs");
  static_assert(BP == 64 || BP == 128, "pixel tile");
  static_assert(KC == 32 || KC == 64, "channel stage");
  static_assert(S >= 2 && S <= 4, "ring depth");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  const uint32_t lds0 = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave % WP, wc = wave / WP;
  // logical block: channel blocks of one range adjacent, so that they run
  // on one XCD and share its L2 copy of the range's pixels
  const int lb = xcd_tile(blockIdx.x, pl.grid);
  const int mb = lb % pl.nmb, rg = lb / pl.nmb;
  // ranges start on multiples of 64 pixels (128-byte aligned row segments:
  // a range starting mid-line costs a third more line fetches per row
  // segment, measured as 4.6 against 6.3-6.5 TB/s of X read) and all but the
  // last hold the same number of pixels
  const int qb = rg * pl.span;
  const int qe = min(qb + pl.span, pl.Q);
  const int ntile = (qe - qb + BP - 1) / BP;
  const int m0 = mb * BC;
  const int HW = a.H * a.W, C = a.C, M = a.M;
  const int nk = C / KC;
  const int total = ntile * nk;               // stages of the block
  if (total <= 0) return;

  // weight DMA offsets at stage 0 (fixed for the block), pixel DMA offsets
  // of the tile the issue cursor is in (bytes; kDmaOutside reads zeros)
  uint32_t xo[IX], wo[IW];
#pragma unroll
  for (int i = 0; i < IW; ++i) {
    const int e = (wave * IW + i) * 64 + lane;
    const int r = e / WPR, jp = e % WPR;
    const int m = m0 + r;
    wo[i] = m < M ? ((uint32_t)m * (uint32_t)C + (uint32_t)(8 * (jp ^ swz_w<KC>(r)))) * 2u : kDmaOutside;
  }
  auto tile_offsets = [&](int t) {
    const int q0 = qb + t * BP, q1 = min(q0 + BP, qe);
#pragma unroll
    for (int i = 0; i < IX; ++i) {
      // LDS position e (in DMA pieces) of this lane: channel row r, 16-byte
      // piece jp / SUB, part jp % SUB; it holds logical piece
      // (jp / SUB) ^ swizzle of the row
      const int e = (wave * IX + i) * 64 + lane;
      const int r = e / (XPR * SUB), jp = e % (XPR * SUB);
      const int q = q0 + 8 * ((jp / SUB) ^ swz_x<BP>(r)) + (jp % SUB) * (PB / 2);
      if (q < q1) {
        const int n = fdiv(pl.hw, q);
        xo[i] = ((uint32_t)(n * C + r) * (uint32_t)HW + (uint32_t)(q - n * HW)) * 2u;
      } else {
        xo[i] = kDmaOutside;
      }
    }
  };
  const uint32_t xstep = (uint32_t)KC * (uint32_t)HW * 2u, wstep = (uint32_t)KC * 2u;
  const u32x4_t xr = buffer_words(a.X, pl.x_bytes);
  const u32x4_t wr = buffer_words(a.Wt, pl.w_bytes);

  // bias of the lane's output channels: branch-free buffer loads issued
  // before any DMA (a channel past M, or no bias at all, reads zero)
  float bv[FC];
  {
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.bias), (short)0, a.bias ? M * 2 : 0, 0x00020000);
    uint32_t braw[FC];
#pragma unroll
    for (int fc = 0; fc < FC; ++fc)
      braw[fc] = __builtin_amdgcn_raw_buffer_load_b16(br, (uint32_t)(m0 + wc * TC + 32 * fc + (lane & 31)) * 2u, 0, 0);
#pragma unroll
    for (int fc = 0; fc < FC; ++fc) bv[fc] = __uint_as_float(braw[fc] << 16);
  }

  // the issue cursor: next stage (tile it, channel stage ik) into slot is
  int it = 0, ik = 0, is = 0, issued = 0;
  tile_offsets(0);
  auto issue_next = [&]() {
    const uint32_t base = lds0 + (uint32_t)(is * SB);
#pragma unroll
    for (int i = 0; i < IX; ++i) {
      if constexpr (PB == 16) dma16(base + (uint32_t)((wave * IX + i) * XI), xo[i] + (uint32_t)ik * xstep, xr);
      else dma4(base + (uint32_t)((wave * IX + i) * XI), xo[i] + (uint32_t)ik * xstep, xr);
    }
#pragma unroll
    for (int i = 0; i < IW; ++i)
      dma16(base + (uint32_t)(XB + (wave * IW + i) * 1024), wo[i] + (uint32_t)ik * wstep, wr);
    ++issued;
    is = is == S - 1 ? 0 : is + 1;
    if (++ik == nk) {
      ik = 0;
      if (++it < ntile) tile_offsets(it);
    }
  };

  // Fragment addresses within a stage.  Pixel (A) fragment fp, k-step s,
  // half h: lane (G = lane/16, j = lane%16) addresses channel row
  // 16s + 8(G/2) + 4h + j/4 at pixels wp*TP + 32fp + 16(G%2) + 4(j%4).
  const int G = lane >> 4, jj = lane & 15;
  const int xrow0 = 8 * (G >> 1) + (jj >> 2);
  const int xswz = swz_x<BP>(xrow0);          // (the swizzle depends on row bits in xrow0 only)
  int xa[FP];
#pragma unroll
  for (int fp = 0; fp < FP; ++fp) {
    const int byte = (wp * TP + 32 * fp + 16 * (G & 1) + 4 * (jj & 3)) * 2;
    xa[fp] = xrow0 * XROW + (((byte >> 4) ^ xswz) << 4) + (byte & 15);
  }
  // weight (B) fragment fc, k-step s: row wc*TC + 32fc + lane%32, piece
  // 2s + lane/32
  int wa[FC], wsw[FC];
#pragma unroll
  for (int fc = 0; fc < FC; ++fc) {
    const int r = wc * TC + 32 * fc + (lane & 31);
    wa[fc] = XB + r * WROW;
    wsw[fc] = (lane >> 5) ^ swz_w<KC>(r);
  }

  f32x16_t acc[FP][FC];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };

  // one stage: the fragments of k-step s+1 are read while the MFMAs of
  // k-step s run (two fragment sets)
  auto compute = [&](int slot) {
    const uint32_t base = lds0 + (uint32_t)(slot * SB);
    u32x4_t af[2][FP], bf[2][FC];
    auto read = [&](int s, int b) {
#pragma unroll
      for (int fp = 0; fp < FP; ++fp) {
        const uint32_t ad = base + (uint32_t)(xa[fp] + 16 * s * XROW);
        const u32x2_t lo = lds_read_tr16(ad), hi = lds_read_tr16(ad + 4 * XROW);
        af[b][fp] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int fc = 0; fc < FC; ++fc)
        bf[b][fc] = lds_read_b128(base + (uint32_t)(wa[fc] + (((2 * s) ^ wsw[fc]) << 4)));
    };
    read(0, 0);
    static_for<NS>([&](auto Sc) {
      constexpr int s = decltype(Sc)::value;
      if constexpr (s + 1 < NS) read(s + 1, (s + 1) & 1);
#pragma unroll
      for (int fp = 0; fp < FP; ++fp)
#pragma unroll
        for (int fc = 0; fc < FC; ++fc) mma32(acc[fp][fc], af[s & 1][fp], bf[s & 1][fc]);
      // the next step's reads interleaved with this step's MFMAs
      constexpr int NM = FP * FC, NR = s + 1 < NS ? 2 * FP + FC : 0;
      constexpr int NMAX = NM > NR ? NM : NR;
#pragma unroll
      for (int i = 0; i < NMAX; ++i) {
        if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Epilogue of tile t.  Lane (l32, kg) holds, for fragment (fp, fc) and
  // group g, channel wc*TC + 32fc + l32 at pixels wp*TP + 32fp + 8g + 4kg
  // .. +3; after the swap of groups (2gp, 2gp+1) it holds pixels
  // wp*TP + 32fp + 16gp + 8kg .. +7.
  const int l32 = lane & 31, kg = lane >> 5;
  uint16_t* Y = (uint16_t*)a.Y;
  const uint16_t* R = (const uint16_t*)a.res;
  auto epilogue = [&](int t) {
    const int q0 = qb + t * BP, q1 = min(q0 + BP, qe);
    with_act(a.act, [&](auto act_k) {
      constexpr int ACT = decltype(act_k)::value;
#pragma unroll
      for (int fc = 0; fc < FC; ++fc) {
        const int m = m0 + wc * TC + 32 * fc + l32;
#pragma unroll
        for (int fp = 0; fp < FP; ++fp)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const int q = q0 + wp * TP + 32 * fp + 16 * gp + 8 * kg;
            const bool ok = m < M && q < q1;
            const f32x16_t& c = acc[fp][fc];
            const int e0 = 8 * gp;          // accumulator index of group 2gp
            uint32_t o[4];
            if constexpr (!RES) {
              uint32_t lo0 = pack_bf16x2(act_c<ACT>(c[e0] + bv[fc]), act_c<ACT>(c[e0 + 1] + bv[fc]));
              uint32_t lo1 = pack_bf16x2(act_c<ACT>(c[e0 + 2] + bv[fc]), act_c<ACT>(c[e0 + 3] + bv[fc]));
              uint32_t hi0 = pack_bf16x2(act_c<ACT>(c[e0 + 4] + bv[fc]), act_c<ACT>(c[e0 + 5] + bv[fc]));
              uint32_t hi1 = pack_bf16x2(act_c<ACT>(c[e0 + 6] + bv[fc]), act_c<ACT>(c[e0 + 7] + bv[fc]));
              swap_halves(lo0, hi0);
              swap_halves(lo1, hi1);
              o[0] = lo0;
              o[1] = lo1;
              o[2] = hi0;
              o[3] = hi1;
            } else {
              // fp32 values through the swap: the residual is added before
              // the activation and the single rounding
              uint32_t v[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) v[i] = __float_as_uint(c[e0 + i] + bv[fc]);
#pragma unroll
              for (int i = 0; i < 4; ++i) swap_halves(v[i], v[i + 4]);
              u32x4_t rr = u32x4_t{0u, 0u, 0u, 0u};
              if (ok) {
                const int n = fdiv(pl.hw, q);
                rr = *(const u32x4_t*)(R + ((int64_t)n * M + m) * HW + (q - n * HW));   // R may be Y: read first
              }
#pragma unroll
              for (int i = 0; i < 4; ++i)
                o[i] = pack_bf16x2(act_c<ACT>(__uint_as_float(v[2 * i]) + __uint_as_float(rr[i] << 16)),
                                   act_c<ACT>(__uint_as_float(v[2 * i + 1]) + __uint_as_float(rr[i] & 0xffff0000u)));
            }
            if (ok) {
              const int n = fdiv(pl.hw, q);
              *(u32x4_t*)(Y + ((int64_t)n * M + m) * HW + (q - n * HW)) = u32x4_t{o[0], o[1], o[2], o[3]};
            }
          }
      }
    });
  };

  // Epilogue of tile t through LDS (no residual): the tile is staged as
  // bf16 channel rows -- in the ring slot its last stage just released, or
  // past the ring where a slot is too small -- and each row segment is
  // written with consecutive lanes on consecutive 16-byte pieces, so that
  // one wave instruction writes whole lines (BP = 128: four rows of 256 B).
  constexpr int EP = BP * 2 + 8;              // bytes per staged row (8 mod 16: conflict-free 8-byte writes)
  constexpr int EB = BC * EP;
  constexpr bool IN_SLOT = EB <= SB;
  auto epilogue_lds = [&](int t, int eslot) {
    const int q0 = qb + t * BP, q1 = min(q0 + BP, qe);
    char* E = smem + (IN_SLOT ? eslot * SB : S * SB);
    if constexpr (IN_SLOT) lds_barrier();     // every wave has read the slot
    with_act(a.act, [&](auto act_k) {
      constexpr int ACT = decltype(act_k)::value;
#pragma unroll
      for (int fc = 0; fc < FC; ++fc) {
        const int col = wc * TC + 32 * fc + l32;
#pragma unroll
        for (int fp = 0; fp < FP; ++fp)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16_t& c = acc[fp][fc];
            const uint32_t lo = pack_bf16x2(act_c<ACT>(c[4 * g] + bv[fc]), act_c<ACT>(c[4 * g + 1] + bv[fc]));
            const uint32_t hi = pack_bf16x2(act_c<ACT>(c[4 * g + 2] + bv[fc]), act_c<ACT>(c[4 * g + 3] + bv[fc]));
            const int px = wp * TP + 32 * fp + 8 * g + 4 * kg;
            *(u32x2_t*)(E + col * EP + px * 2) = u32x2_t{lo, hi};
          }
      }
    });
    lds_barrier();
    // runs of V pixels of one channel row (HW % V == 0: a run never
    // straddles two images), consecutive lanes on consecutive runs
    auto store_runs = [&](auto Vc) {
      constexpr int V = decltype(Vc)::value, RPR = BP / V;
      constexpr int ITEMS = BC * RPR;
#pragma unroll 2
      for (int it = tid; it < ITEMS; it += kThreads) {
        const int row = it / RPR, pc = it - (it / RPR) * RPR;
        const int m = m0 + row, q = q0 + V * pc;
        if (m < M && q < q1) {
          const int n = fdiv(pl.hw, q);
          const char* src = E + row * EP + pc * V * 2;
          uint16_t* dst = Y + ((int64_t)n * M + m) * HW + (q - n * HW);
          if constexpr (V == 8) {
            const u32x2_t p0 = *(const u32x2_t*)src, p1 = *(const u32x2_t*)(src + 8);
            *(u32x4_t*)dst = u32x4_t{p0[0], p0[1], p1[0], p1[1]};
          } else if constexpr (V == 4) {
            *(u32x2_t*)dst = *(const u32x2_t*)src;
          } else if constexpr (V == 2) {
            *(uint32_t*)dst = *(const uint32_t*)src;
          } else {
            *dst = *(const uint16_t*)src;
          }
        }
      }
    };
    switch (pl.V) {
      case 8: store_runs(std::integral_constant<int, 8>{}); break;
      case 4: store_runs(std::integral_constant<int, 4>{}); break;
      case 2: store_runs(std::integral_constant<int, 2>{}); break;
      default: store_runs(std::integral_constant<int, 1>{}); break;
    }
    // (the next stage's wait includes lgkmcnt(0) before its barrier: the
    // staging reads are done before any DMA reuses the slot)
  };

  // The ring.  Stage j lives in slot j % S; S-1 stages are issued ahead.
  // The wait before stage j counts only the DMA instructions issued after
  // it; the epilogue's stores (also counted by vmcnt) are younger still, so
  // they only make the wait more conservative.
#pragma unroll
  for (int k = 0; k < S - 1; ++k)
    if (issued < total) issue_next();
  int slot = 0, ct = 0, ck = 0;
  zero_acc();
  for (int j = 0; j < total; ++j) {
    wait_dma_barrier_rt<D, S - 2>(total - 1 - j);
    if (issued < total) issue_next();     // into the slot read by stage j-1
    const int cs = slot;
    compute(cs);
    slot = slot == S - 1 ? 0 : slot + 1;
    if (++ck == nk) {
      if constexpr (RES) epilogue(ct);
      else epilogue_lds(ct, cs);
      zero_acc();
      ck = 0;
      ++ct;
    }
  }
}

// LDS bytes of a configuration: the ring, plus the epilogue's staging tile
// where a ring slot cannot hold it (no residual)
template <int BP, int BC, int KC, int S, bool RES>
constexpr int lds_bytes() {
  constexpr int ring = S * (KC * BP * 2 + BC * KC * 2);
  constexpr int stage = BC * (BP * 2 + 8);
  return RES || stage <= KC * BP * 2 + BC * KC * 2 ? ring : ring + stage;
}

template <int BP, int BC, int KC, int S, int WP>
int launch(const ConvArgs& a, const PwdPlan& p, hipStream_t s) {
  dim3 grid(p.grid, 1, 1);
  constexpr int LR = lds_bytes<BP, BC, KC, S, true>(), L = lds_bytes<BP, BC, KC, S, false>();
  if (p.PB == 4)   // (the planner gives a residual only 16-byte pieces)
    hipLaunchKernelGGL((conv1x1_dma<BP, BC, KC, S, WP, 4, false>), grid, dim3(kThreads), L, s, a, p);
  else if (a.res)
    hipLaunchKernelGGL((conv1x1_dma<BP, BC, KC, S, WP, 16, true>), grid, dim3(kThreads), LR, s, a, p);
  else
    hipLaunchKernelGGL((conv1x1_dma<BP, BC, KC, S, WP, 16, false>), grid, dim3(kThreads), L, s, a, p);
  return (int)hipGetLastError();
}

}  // namespace pwd

}  // namespace ox
