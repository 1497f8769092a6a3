// conv_pw.hpp -- pointwise (1x1, stride 1, unpadded) convolution on NCHW,
// bf16, as one GEMM over all pixels of the batch (instantiated by
// k_conv_pw_*.hip).
//
// Y[n, m, p] = act(bias[m] + sum_c W[m, c] * X[n, c, p]).  The pixels of the
// batch are flattened (q = n*HW + p) and a tile is BN consecutive pixels x
// BM output channels.  For each chunk of KC input channels a block
//   * stages the pixels channel-contiguous in LDS: one (2*KC + 16)-byte row
//     per pixel (KC channels plus 16 bytes of bank padding).  A staging unit
//     is P consecutive pixels x 8 channels: 8 loads of P elements, with
//     consecutive lanes on consecutive pixel groups (coalesced along the
//     plane), repacked by pixel into 16-byte row pieces;
//   * stages the weight rows W[m, c0 .. c0+KC) with 16-byte loads (the ONNX
//     layout already has each row's channels contiguous);
//   * runs KC/16 k-steps of FP x FC v_mfma_f32_32x32x16_bf16 per wave, both
//     fragments single 128-bit LDS reads, read two steps ahead and
//     interleaved with the MFMAs.
// Blocks are persistent: each walks a strided sequence of work units and
// loads the next unit's first chunk while the current one finishes its
// MFMAs and epilogue.  A work unit is a tile, or -- when there are too few
// tiles to occupy the chip -- one of S slices of a tile's channel range
// (split-K): a slice writes its fp32 partial tile to a workspace and
// conv1x1_reduce adds the S partials in slice order (deterministic) and runs
// the epilogue.  The epilogue (bias, activation, bf16 rounding) stages the
// tile in LDS as [channel][pixel] and writes each channel's pixels with
// aligned vector stores.
#pragma once

#include "engine.hpp"

namespace ox {

namespace pw {

// Bias, activation and bf16 conversion of one tile held in the MFMA
// accumulators of the block's four waves, staged through LDS and stored as
// channel runs.  Lane (l32, kg) of wave (wm, wn) holds, for each (fp, fc),
// channel 32*(wm*FC + fc) + l32 at pixel slots 32*(wn*FP + fp) + 8*g + 4*kg
// + (0..3).  The caller has synchronised the block: LDS is free.
template <int WM, int WN, int FP, int FC>
__device__ __forceinline__ void store_tile(const ConvArgs& a, const PwPlan& pl, char* smem,
                                           const uint16_t* Bv, const f32x16_t (&acc)[FP][FC], int q0,
                                           int m0) {
  constexpr int BM = 32 * WM * FC, BN = 32 * WN * FP;
  constexpr int EROW = BN + 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l32 = lane & 31, kg = lane >> 5;
  const int HW = a.H * a.W, M = a.M, Q = a.N * HW;
  uint16_t* E = (uint16_t*)smem;
  float bv[FC];
#pragma unroll
  for (int fc = 0; fc < FC; ++fc) {
    const int m = m0 + wm * FC * 32 + fc * 32 + l32;
    bv[fc] = (Bv && m < M) ? bf16_to_f32(Bv[m]) : 0.0f;
  }
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int fc = 0; fc < FC; ++fc) {
      const int ml = wm * FC * 32 + fc * 32 + l32;
#pragma unroll
      for (int fp = 0; fp < FP; ++fp) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int slot = (wn * FP + fp) * 32 + 8 * g + 4 * kg;
          const f32x16_t& c = acc[fp][fc];
          const uint32_t lo = pack_bf16x2(act_c<ACT>(c[4 * g + 0] + bv[fc]),
                                          act_c<ACT>(c[4 * g + 1] + bv[fc]));
          const uint32_t hi = pack_bf16x2(act_c<ACT>(c[4 * g + 2] + bv[fc]),
                                          act_c<ACT>(c[4 * g + 3] + bv[fc]));
          *(u32x2_t*)(E + ml * EROW + slot) = u32x2_t{lo, hi};
        }
      }
    }
  });
  __syncthreads();
  uint16_t* Y = (uint16_t*)a.Y;
  const int mvalid = min(BM, M - m0);
  const int V = pl.V;                      // HW % V == 0 and Y is 2V-byte aligned
  const int per_row = BN / V;
  const int items = mvalid * per_row;
  for (int it = tid; it < items; it += kThreads) {
    const int m = it / per_row;
    const int e = (it - m * per_row) * V;
    const int q = q0 + e;
    if (q >= Q) continue;
    const int n = q / HW;
    const uint16_t* src = E + m * EROW + e;
    uint16_t* dst = Y + ((int64_t)n * M + m0 + m) * HW + (q - n * HW);
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

// Workspace layout of split-K partials: unit (tile, slice) owns
// kThreads * FP*FC*4 float4 values, stored [float4 index][thread] so that
// both the writer and the reducer access it fully coalesced.
template <int FP, int FC>
__device__ __forceinline__ f32x4_t* partial_base(float* ws, int64_t unit) {
  return (f32x4_t*)ws + unit * (int64_t)(kThreads * FP * FC * 4);
}

template <int WM, int WN, int FP, int FC, int KC, int P>
__global__ __launch_bounds__(kThreads, 2) void conv1x1_bf16(const ConvArgs a, const PwPlan pl) {
  constexpr int BM = 32 * WM * FC;          // output channels per tile
  constexpr int BN = 32 * WN * FP;          // pixels per tile
  constexpr int ROW = KC * 2 + 16;          // bytes per staged row
  constexpr int NG = BN / P;                // pixel groups per tile
  constexpr int XU = (KC / 8) * NG;         // pixel staging units per chunk
  constexpr int XUPT = (XU + kThreads - 1) / kThreads;
  constexpr int WPR = KC / 8;               // 16-byte weight pieces per row
  constexpr int WU = BM * WPR;
  constexpr int WUPT = (WU + kThreads - 1) / kThreads;
  constexpr int NS = KC / 16;               // k-steps per chunk
  static_assert(WM * WN == 4, "four waves");
  static_assert(BN % P == 0 && KC % 32 == 0, "tile shape");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // two operand buffers: chunk k+1 is staged into one while chunk k's MFMAs
  // read the other
  constexpr int BUF = (BM + BN) * ROW;
  auto As = [&](int b) { return smem + b * BUF; };             // weights [BM][ROW]
  auto Xs = [&](int b) { return smem + b * BUF + BM * ROW; };  // pixels  [BN][ROW]
  // the bias vector, raw bf16, beyond both the operand buffers and the
  // epilogue's staging area: staged once per block with the first chunk (as
  // the 32-bit words that hold it, from its aligned-down address), so that
  // no epilogue waits on a global load and no load is carried across units
  uint32_t* Bw = (uint32_t*)(smem + pl.lds - pl.bias_lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l32 = lane & 31, kg = lane >> 5;
  const int tiles = pl.npb * pl.nmb;
  const int S = pl.splits, cps = pl.cps;    // slices per tile, chunks per slice
  const int units = tiles * S;
  const int HW = a.H * a.W, C = a.C, M = a.M;
  const int Q = a.N * HW;
  const int nchunks = C / KC;
  const uint16_t* Xg = (const uint16_t*)a.X;
  const uint16_t* Wg = (const uint16_t*)a.Wt;

  // Block b runs units b, b + G, b + 2G, ... (G = grid size, a multiple of
  // the XCD count when below the unit count), so a block stays on one XCD and
  // xcd_tile keeps each XCD on one contiguous range of logical units (the
  // slices of a tile adjacent, then the channel blocks of a pixel block).
  int u = blockIdx.x;
  if (u >= units) return;
  int pb, m0, c_lo, c_hi, unit_id;
  auto decode = [&](int uu) {
    unit_id = xcd_tile(uu, units);
    const int tile = unit_id / S;
    const int slice = unit_id - tile * S;
    pb = tile / pl.nmb;
    m0 = (tile - pb * pl.nmb) * BM;
    c_lo = slice * cps;
    c_hi = min(nchunks, c_lo + cps);
  };

  // this thread's pixel staging units: element offset of the first value and
  // LDS offset of its first row piece; units and weight pieces that fall
  // outside the tensors load from offset 0 and store zeros (loads are never
  // predicated: a register that a load may or may not write would force the
  // wave to wait on every load in flight before reusing it)
  int x_goff[XUPT], x_lds[XUPT];
  int w_goff[WUPT], w_lds[WUPT];
  uint32_t x_ok = 0, w_ok = 0;   // bit k: unit / piece k is inside the tensor
#pragma unroll
  for (int k = 0; k < XUPT; ++k) {
    const int v = tid + k * kThreads;
    x_lds[k] = v < XU ? (v % NG) * P * ROW + (v / NG) * 16 : 0;
  }
#pragma unroll
  for (int k = 0; k < WUPT; ++k) {
    const int v = tid + k * kThreads;
    w_lds[k] = (v / WPR) * ROW + (v % WPR) * 16;
  }
  auto tile_offsets = [&]() {
    const int q0 = pb * BN;
    x_ok = w_ok = 0;
#pragma unroll
    for (int k = 0; k < XUPT; ++k) {
      const int v = tid + k * kThreads;
      const int oct = v / NG, g = v - (v / NG) * NG;
      const int q = q0 + g * P;
      const bool ok = v < XU && q < Q;
      const int n = ok ? q / HW : 0;
      x_goff[k] = ok ? (n * C + oct * 8) * HW + (q - n * HW) : 0;
      x_ok |= (ok ? 1u : 0u) << k;
    }
#pragma unroll
    for (int k = 0; k < WUPT; ++k) {
      const int v = tid + k * kThreads;
      const int m = v / WPR, j = v - (v / WPR) * WPR;
      const bool ok = v < WU && m0 + m < M;
      w_goff[k] = ok ? (m0 + m) * C + j * 8 : 0;
      w_ok |= (ok ? 1u : 0u) << k;
    }
  };

  const int pbase = (wn * FP * 32 + l32) * ROW + kg * 16;   // + f*32*ROW
  const int wbase = (wm * FC * 32 + l32) * ROW + kg * 16;   // + f*32*ROW

  f32x16_t acc[FP][FC];
  // P = 1: one bf16 per load; P = 2: one dword; P = 4: two dwords
  constexpr int XR = P == 4 ? 2 : 1;
  uint32_t xreg[XUPT][8][XR];
  u32x4_t wreg[WUPT];
  constexpr int BWPT = 4;          // bias words per thread in the first round
  const uint16_t* bias = (const uint16_t*)a.bias;
  const uintptr_t baddr = (uintptr_t)bias;
  const int boff = (int)(baddr & 3);                       // byte offset of bias[0] in its word
  const uint32_t* bwords = (const uint32_t*)(baddr & ~(uintptr_t)3);
  const int nbw = (bias && S == 1) ? (boff + 2 * M + 3) / 4 : 0;
  const uint16_t* Bv = nbw ? (const uint16_t*)((const char*)Bw + boff) : nullptr;
  uint32_t bwv[BWPT];
  if (nbw > 0) {
#pragma unroll
    for (int k = 0; k < BWPT; ++k) bwv[k] = bwords[min(tid + k * kThreads, nbw - 1)];
  }
  auto store_bias = [&]() {
#pragma unroll
    for (int k = 0; k < BWPT; ++k)
      if (tid + k * kThreads < nbw) Bw[tid + k * kThreads] = bwv[k];
    for (int i = tid + BWPT * kThreads; i < nbw; i += kThreads) Bw[i] = bwords[i];
  };

  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int k = 0; k < WUPT; ++k) wreg[k] = *(const u32x4_t*)(Wg + w_goff[k] + c0);
#pragma unroll
    for (int k = 0; k < XUPT; ++k) {
      const uint16_t* src = Xg + x_goff[k] + c0 * HW;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        if constexpr (P == 1) {
          xreg[k][ch][0] = src[ch * HW];
        } else if constexpr (P == 2) {
          xreg[k][ch][0] = *(const uint32_t*)(src + ch * HW);
        } else {
          const u32x2_t v = *(const u32x2_t*)(src + ch * HW);
          xreg[k][ch][0] = v[0];
          xreg[k][ch][1] = v[1];
        }
      }
    }
  };

  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int k = 0; k < WUPT; ++k)
      if (k * kThreads + kThreads <= WU || tid + k * kThreads < WU)
        *(u32x4_t*)(As(buf) + w_lds[k]) = ((w_ok >> k) & 1) ? wreg[k] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < XUPT; ++k) {
      if (k * kThreads + kThreads <= XU || tid + k * kThreads < XU) {
#pragma unroll
        for (int e = 0; e < P; ++e) {
          // pixel e of the unit: bf16 number e of each channel's loaded P
          uint32_t d[4];
          const bool ok = (x_ok >> k) & 1;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = ok ? xreg[k][2 * j][e >> 1] : 0u, hi = ok ? xreg[k][2 * j + 1][e >> 1] : 0u;
            if constexpr (P == 1) d[j] = (lo & 0xffffu) | (hi << 16);
            else if ((e & 1) == 0) d[j] = (lo & 0xffffu) | (hi << 16);
            else d[j] = (lo >> 16) | (hi & 0xffff0000u);
          }
          *(u32x4_t*)(Xs(buf) + x_lds[k] + e * ROW) = u32x4_t{d[0], d[1], d[2], d[3]};
        }
      }
    }
  };

  decode(u);
  tile_offsets();
  load_chunk(c_lo * KC);
  bool first_unit = true;
  for (;;) {
    const int cur_pb = pb, cur_m0 = m0, cur_lo = c_lo, cur_hi = c_hi, cur_unit = unit_id;
    const int next = u + (int)gridDim.x;
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // the registers hold chunk cur_lo; after a chunk is stored they are
    // refilled with the next chunk of this unit or, after its last, with the
    // next unit's first chunk
    auto load_after = [&](int c) {
      if (c < cur_hi) {
        load_chunk(c * KC);
      } else if (next < units) {
        decode(next);
        tile_offsets();
        load_chunk(c_lo * KC);
      }
    };
    __syncthreads();                 // LDS is free: previous MFMAs and epilogue are done
    if (first_unit) store_bias();
    first_unit = false;
    store_chunk(0);
    load_after(cur_lo + 1);
    __syncthreads();
    for (int chunk = cur_lo; chunk < cur_hi; ++chunk) {
      const int buf = (chunk - cur_lo) & 1;
      const char* Xb = Xs(buf);
      const char* Ab = As(buf);
      u32x4_t pf[3][FP], wf[3][FC];
      auto read_frags = [&](int s, int fb) {
#pragma unroll
        for (int f = 0; f < FP; ++f) pf[fb][f] = *(const u32x4_t*)(Xb + pbase + f * 32 * ROW + s * 32);
#pragma unroll
        for (int f = 0; f < FC; ++f) wf[fb][f] = *(const u32x4_t*)(Ab + wbase + f * 32 * ROW + s * 32);
      };
      read_frags(0, 0);
      if (NS > 1) read_frags(1, 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bool ahead = s + 2 < NS;
        if (ahead) read_frags(s + 2, (s + 2) % 3);
#pragma unroll
        for (int fp = 0; fp < FP; ++fp)
#pragma unroll
          for (int fc = 0; fc < FC; ++fc) mma32(acc[fp][fc], pf[s % 3][fp], wf[s % 3][fc]);
        constexpr int NM = FP * FC, NR = FP + FC;
#pragma unroll
        for (int i = 0; i < (NM > NR ? NM : NR); ++i) {
          if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          if (ahead && i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (chunk + 1 < cur_hi) {
        store_chunk(buf ^ 1);        // the other buffer: its last reader finished before the previous barrier
        load_after(chunk + 2);
      }
      __syncthreads();
    }
    if (S == 1) {
      store_tile<WM, WN, FP, FC>(a, pl, smem, Bv, acc, cur_pb * BN, cur_m0);
    } else {
      f32x4_t* dst = partial_base<FP, FC>(pl.ws, cur_unit) + tid;
#pragma unroll
      for (int fp = 0; fp < FP; ++fp)
#pragma unroll
        for (int fc = 0; fc < FC; ++fc)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            dst[((fp * FC + fc) * 4 + g) * kThreads] =
                f32x4_t{acc[fp][fc][4 * g], acc[fp][fc][4 * g + 1], acc[fp][fc][4 * g + 2],
                        acc[fp][fc][4 * g + 3]};
    }
    if (next >= units) break;
    u = next;
  }
}

// Second pass of split-K.  One block per (tile, wave of the first pass):
// its 256 threads split that wave's 64 x FP*FC*4 float4 partial values four
// ways (more loads in flight per CU), add the S slices in slice order, apply
// bias and activation, stage the 32*FC x 32*FP sub-tile in LDS as
// [channel][pixel] and write the channel runs.
template <int WM, int WN, int FP, int FC>
__global__ __launch_bounds__(kThreads) void conv1x1_reduce(const ConvArgs a, const PwPlan pl) {
  constexpr int BN = 32 * WN * FP, BM = 32 * WM * FC;
  constexpr int SUBM = 32 * FC, SUBN = 32 * FP, EROW = SUBN + 8;
  constexpr int NV = FP * FC * 4;           // float4 values per lane of the first pass
  constexpr int PER = NV / 4;               // of those, per thread here
  static_assert(NV % 4 == 0, "four threads per lane");
  __shared__ __attribute__((aligned(16))) uint16_t E[SUBM * EROW];
  const int t = blockIdx.x >> 2, w = blockIdx.x & 3;
  const int wm = w / WN, wn = w - (w / WN) * WN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, part = tid >> 6;     // first-pass lane, quarter of its values
  const int l32 = lane & 31, kg = lane >> 5;
  f32x4_t sum[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) sum[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int s = 0; s < pl.splits; ++s) {
    const f32x4_t* src = partial_base<FP, FC>(pl.ws, (int64_t)t * pl.splits + s) + w * 64 + lane;
#pragma unroll
    for (int k = 0; k < PER; ++k) sum[k] += src[(part * PER + k) * kThreads];
  }
  const int pb = t / pl.nmb;
  const int q0 = pb * BN + wn * SUBN, m0 = (t - pb * pl.nmb) * BM + wm * SUBM;
  const int HW = a.H * a.W, M = a.M, Q = a.N * HW;
  const uint16_t* bias = (const uint16_t*)a.bias;
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = part * PER + k;             // value index (fp*FC + fc)*4 + g
      const int g = i & 3, fc = (i >> 2) % FC, fp = (i >> 2) / FC;
      const int m = m0 + fc * 32 + l32;
      const float bv = (bias && m < M) ? bf16_to_f32(bias[m]) : 0.0f;
      const uint32_t lo = pack_bf16x2(act_c<ACT>(sum[k][0] + bv), act_c<ACT>(sum[k][1] + bv));
      const uint32_t hi = pack_bf16x2(act_c<ACT>(sum[k][2] + bv), act_c<ACT>(sum[k][3] + bv));
      *(u32x2_t*)(E + (fc * 32 + l32) * EROW + fp * 32 + 8 * g + 4 * kg) = u32x2_t{lo, hi};
    }
  });
  __syncthreads();
  if (m0 >= M) return;
  uint16_t* Y = (uint16_t*)a.Y;
  const int mvalid = min(SUBM, M - m0);
  const int V = pl.V;
  const int per_row = SUBN / V;
  for (int it = tid; it < mvalid * per_row; it += kThreads) {
    const int m = it / per_row;
    const int e = (it - m * per_row) * V;
    const int q = q0 + e;
    if (q >= Q) continue;
    const int n = q / HW;
    const uint16_t* src = E + m * EROW + e;
    uint16_t* dst = Y + ((int64_t)n * M + m0 + m) * HW + (q - n * HW);
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

template <int WM, int WN, int FP, int KC>
int launch_fp(const ConvArgs& a, const PwPlan& p, hipStream_t s) {
  constexpr int FC = 2;
  dim3 grid(p.grid, 1, 1);
  switch (p.P) {
    case 4:
      hipLaunchKernelGGL((conv1x1_bf16<WM, WN, FP, FC, KC, 4>), grid, dim3(kThreads), p.lds, s, a, p);
      break;
    case 2:
      hipLaunchKernelGGL((conv1x1_bf16<WM, WN, FP, FC, KC, 2>), grid, dim3(kThreads), p.lds, s, a, p);
      break;
    default:
      hipLaunchKernelGGL((conv1x1_bf16<WM, WN, FP, FC, KC, 1>), grid, dim3(kThreads), p.lds, s, a, p);
      break;
  }
  if (p.splits > 1)
    hipLaunchKernelGGL((conv1x1_reduce<WM, WN, FP, FC>), dim3(p.npb * p.nmb * 4), dim3(kThreads), 0, s, a, p);
  return (int)hipGetLastError();
}

template <int WM, int WN, int KC>
int launch_cfg(const ConvArgs& a, const PwPlan& p, hipStream_t s) {
  return p.FP == 1 ? launch_fp<WM, WN, 1, KC>(a, p, s) : launch_fp<WM, WN, 2, KC>(a, p, s);
}

}  // namespace pw

// launch_pw_<WM>_<KC>: tiles of 64*WM channels x 32*(4/WM)*FP pixels, KC
// input channels per chunk (wider chunks would not fit the staging
// registers next to the accumulators)
int launch_pw_1_32(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_1_64(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_2_32(const ConvArgs& a, const PwPlan& p, void* s);
int launch_pw_2_64(const ConvArgs& a, const PwPlan& p, void* s);

}  // namespace ox
