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
// the epilogue from its registers.  The first pass's epilogue (bias,
// activation, bf16 rounding) stages the tile in LDS as [channel][pixel] and
// writes each channel's pixels with aligned vector stores.
#pragma once

#include "engine.hpp"

namespace ox {

namespace pw {

// The epilogue with a residual input R (Y's shape and type): the tile's fp32
// values acc + bias are staged in LDS as [channel][pixel], then each
// channel's run of V pixels is read back, R's matching run added (one vector
// load, coalesced along the plane), the activation applied and the result
// stored: Y = act((acc + bias) + R).  R may be Y itself (each element is
// read before it is written, by the same thread).  The caller has
// synchronised the block: LDS is free.
template <int WM, int WN, int FP, int FC>
__device__ __forceinline__ void store_tile_res(const ConvArgs& a, const PwPlan& pl, char* smem,
                                               const float (&bv)[FC], const f32x16_t (&acc)[FP][FC],
                                               int q0, int m0) {
  constexpr int BM = 32 * WM * FC, BN = 32 * WN * FP;
  constexpr int EROW = BN + 4;             // floats per staged channel row
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int l32 = lane & 31, kg = lane >> 5;
  const int HW = a.H * a.W, M = a.M, Q = a.N * HW;
  float* E = (float*)smem;
#pragma unroll
  for (int fc = 0; fc < FC; ++fc) {
    const int ml = wm * FC * 32 + fc * 32 + l32;
#pragma unroll
    for (int fp = 0; fp < FP; ++fp) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int slot = (wn * FP + fp) * 32 + 8 * g + 4 * kg;
        const f32x16_t& c = acc[fp][fc];
        *(f32x4_t*)(E + ml * EROW + slot) =
            f32x4_t{c[4 * g] + bv[fc], c[4 * g + 1] + bv[fc], c[4 * g + 2] + bv[fc], c[4 * g + 3] + bv[fc]};
      }
    }
  }
  __syncthreads();
  uint16_t* Y = (uint16_t*)a.Y;
  const uint16_t* R = (const uint16_t*)a.res;
  const int mvalid = min(BM, M - m0);
  const int per_row_v = BN / pl.V;
  const int items = mvalid * per_row_v;
  // Runs are handled 4 per thread at a time: the 4 residual loads are all
  // issued before the first store (R may be Y itself, so the compiler could
  // not move a load above an earlier store on its own).
  auto run = [&](auto Vc, auto act_k) {
    constexpr int V = decltype(Vc)::value, ACT = decltype(act_k)::value;
    constexpr int NW = V >= 2 ? V / 2 : 1;          // 32-bit residual words per run
    constexpr int G = 4;
    const int per_row = BN / V;
    for (int base = tid; base < items; base += G * kThreads) {
      uint32_t rw[G][NW];
      int off[G];                                   // (the plan keeps Y below 2^31 elements)
      int srcv[G];
      bool ok[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int it = base + u * kThreads;
        const int m = it / per_row;
        const int e = (it - m * per_row) * V;
        const int q = q0 + e;
        ok[u] = it < items && q < Q;
        const int n = ok[u] ? q / HW : 0;
        off[u] = ok[u] ? (n * M + m0 + m) * HW + (q - n * HW) : 0;
        srcv[u] = m * EROW + e;
        if constexpr (V == 8) {
          const u32x4_t r = ok[u] ? *(const u32x4_t*)(R + off[u]) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
          for (int j = 0; j < 4; ++j) rw[u][j] = r[j];
        } else if constexpr (V == 4) {
          const u32x2_t r = ok[u] ? *(const u32x2_t*)(R + off[u]) : u32x2_t{0u, 0u};
          rw[u][0] = r[0];
          rw[u][1] = r[1];
        } else if constexpr (V == 2) {
          rw[u][0] = ok[u] ? *(const uint32_t*)(R + off[u]) : 0u;
        } else {
          rw[u][0] = ok[u] ? (uint32_t)R[off[u]] : 0u;
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (!ok[u]) continue;
        const float* src = E + srcv[u];
        if constexpr (V == 1) {
          Y[off[u]] = f32_to_bf16(act_c<ACT>(src[0] + __uint_as_float(rw[u][0] << 16)));
        } else {
          uint32_t o[NW];
#pragma unroll
          for (int j = 0; j < NW; ++j)
            o[j] = pack_bf16x2(act_c<ACT>(src[2 * j] + __uint_as_float(rw[u][j] << 16)),
                               act_c<ACT>(src[2 * j + 1] + __uint_as_float(rw[u][j] & 0xffff0000u)));
          if constexpr (V == 8) *(u32x4_t*)(Y + off[u]) = u32x4_t{o[0], o[1], o[2], o[3]};
          else if constexpr (V == 4) *(u32x2_t*)(Y + off[u]) = u32x2_t{o[0], o[1]};
          else *(uint32_t*)(Y + off[u]) = o[0];
        }
      }
    }
  };
  with_act(a.act, [&](auto act_k) {
    switch (pl.V) {                        // HW % V == 0, Y and R 2V-byte aligned
      case 8: run(std::integral_constant<int, 8>{}, act_k); break;
      case 4: run(std::integral_constant<int, 4>{}, act_k); break;
      case 2: run(std::integral_constant<int, 2>{}, act_k); break;
      default: run(std::integral_constant<int, 1>{}, act_k); break;
    }
  });
}

// Bias, activation and bf16 conversion of one tile held in the MFMA
// accumulators of the block's four waves, staged through LDS and stored as
// channel runs.  Lane (l32, kg) of wave (wm, wn) holds, for each (fp, fc),
// channel 32*(wm*FC + fc) + l32 at pixel slots 32*(wn*FP + fp) + 8*g + 4*kg
// + (0..3).  The caller has synchronised the block: LDS is free.
template <int WM, int WN, int FP, int FC, bool RES>
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
  if constexpr (RES) {
    store_tile_res<WM, WN, FP, FC>(a, pl, smem, bv, acc, q0, m0);
    return;
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

// Raw buffer resource over [p, p + bytes): a load whose offset lies beyond
// the range returns zeros, which stands in for the zero padding of partial
// tiles (rows past M, pixels past the batch) with no per-load predicate.
constexpr uint32_t kOutside = 0x80000000u;    // an offset past any tensor the kernel takes
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int WM, int WN, int FP, int FC, int KC, int P, bool RES>
__global__ __launch_bounds__(kThreads, (KC == 32 && !RES) ? 3 : 2) void conv1x1_bf16(const ConvArgs a, const PwPlan pl) {
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
  // register sets of loaded chunks: two for 64-channel chunks; one for
  // 32-channel chunks, whose blocks are small enough to run three per CU
  // (a second set would cost that occupancy).  The residual epilogue's
  // fp32 staging leaves room for two blocks per CU whatever the chunk, and
  // its registers take the place of the second set.
  constexpr int NSET = (KC == 64 && !RES) ? 2 : 1;
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
  // (the plan keeps both tensors below 2^30 bytes, so that no offset of a
  // unit past the tensor's end wraps around 2^32)
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(a.X, (uint32_t)Q * (uint32_t)C * 2u);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.Wt, (uint32_t)M * (uint32_t)C * 2u);

  // Block b runs units b, b + G, b + 2G, ... (G = grid size, a multiple of
  // the XCD count when below the unit count), so a block stays on one XCD and
  // xcd_tile keeps each XCD on one contiguous range of logical units (the
  // slices of a tile adjacent, then the channel blocks of a pixel block).
  if ((int)blockIdx.x >= units) return;
  struct Unit {
    int id, pb, m0, lo, hi;   // logical unit, pixel block, first channel, chunk range
  };
  auto decode = [&](int uu) {
    Unit d;
    d.id = xcd_tile(uu, units);
    const int tile = d.id / S;
    const int slice = d.id - tile * S;
    d.pb = tile / pl.nmb;
    d.m0 = (tile - d.pb * pl.nmb) * BM;
    d.lo = slice * cps;
    d.hi = min(nchunks, d.lo + cps);
    return d;
  };

  // The block's chunks form one stream (unit after unit).  Stream position j
  // is loaded into register set j % NSET, NSET positions ahead of its use:
  // while chunk j's MFMAs run, chunk j+1 is staged from its registers into
  // the other LDS buffer and (two sets) the loads of chunk j+2 are in
  // flight.  The load cursor runs ahead of the compute cursor and crosses
  // into the next unit on its own.
  //
  // Staging units of this thread: byte offset of the first value in X (or in
  // W) at chunk 0 and LDS offset of its first row piece.  Units past the
  // tile's pixels or channels read beyond the tensor and get zeros.
  uint32_t x_off[XUPT], w_off[WUPT];
  int x_lds[XUPT], w_lds[WUPT];
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
  auto tile_offsets = [&](int pb, int m0) {
    const int q0 = pb * BN;
#pragma unroll
    for (int k = 0; k < XUPT; ++k) {
      const int v = tid + k * kThreads;
      const int oct = v / NG, g = v - (v / NG) * NG;
      const int q = q0 + g * P;
      const int n = q / HW;                 // n >= N past the batch: beyond X
      x_off[k] = v < XU ? ((uint32_t)(n * C + oct * 8) * (uint32_t)HW + (uint32_t)(q - n * HW)) * 2u : kOutside;
    }
#pragma unroll
    for (int k = 0; k < WUPT; ++k) {
      const int v = tid + k * kThreads;
      const int m = v / WPR, j = v - (v / WPR) * WPR;
      // rows m0 + m >= M lie beyond W
      w_off[k] = v < WU ? ((uint32_t)(m0 + m) * (uint32_t)C + (uint32_t)(j * 8)) * 2u : kOutside;
    }
  };

  const int pbase = (wn * FP * 32 + l32) * ROW + kg * 16;   // + f*32*ROW
  const int wbase = (wm * FC * 32 + l32) * ROW + kg * 16;   // + f*32*ROW

  f32x16_t acc[FP][FC];
  // P = 1: one bf16 per load; P = 2: one dword; P = 4: two dwords
  constexpr int XR = P == 4 ? 2 : 1;
  uint32_t xreg[NSET][XUPT][8][XR];
  u32x4_t wreg[NSET][WUPT];
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

  // global loads of chunk c0 of the load cursor's unit into register set R
  auto load_chunk = [&](auto Rc, int c0) {
    constexpr int R = decltype(Rc)::value % NSET;
    const uint32_t wc = (uint32_t)c0 * 2u;
#pragma unroll
    for (int k = 0; k < WUPT; ++k) wreg[R][k] = __builtin_amdgcn_raw_buffer_load_b128(wr, w_off[k] + wc, 0, 0);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      const uint32_t xc = (uint32_t)(c0 + ch) * (uint32_t)HW * 2u;
#pragma unroll
      for (int k = 0; k < XUPT; ++k) {
        if constexpr (P == 1) {
          xreg[R][k][ch][0] = __builtin_amdgcn_raw_buffer_load_b16(xr, x_off[k] + xc, 0, 0);
        } else if constexpr (P == 2) {
          xreg[R][k][ch][0] = __builtin_amdgcn_raw_buffer_load_b32(xr, x_off[k] + xc, 0, 0);
        } else {
          const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(xr, x_off[k] + xc, 0, 0);
          xreg[R][k][ch][0] = v[0];
          xreg[R][k][ch][1] = v[1];
        }
      }
    }
  };

  // LDS stores of register set R into operand buffer B: piece i of NPC
  // (weight pieces first, then one piece per pixel of each staging unit)
  constexpr int NPC = WUPT + XUPT * P;
  auto store_piece = [&](auto Rc, auto Bc, auto Ic) {
    constexpr int R = decltype(Rc)::value % NSET, B = decltype(Bc)::value, I = decltype(Ic)::value;
    if constexpr (I < WUPT) {
      constexpr int k = I;
      if (k * kThreads + kThreads <= WU || tid + k * kThreads < WU)
        *(u32x4_t*)(As(B) + w_lds[k]) = wreg[R][k];
    } else {
      constexpr int k = (I - WUPT) / P, e = (I - WUPT) % P;
      if (k * kThreads + kThreads <= XU || tid + k * kThreads < XU) {
        // pixel e of the unit: bf16 number e of each channel's loaded P
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = xreg[R][k][2 * j][e >> 1], hi = xreg[R][k][2 * j + 1][e >> 1];
          d[j] = __builtin_amdgcn_perm(hi, lo, (P == 1 || (e & 1) == 0) ? 0x05040100u : 0x07060302u);
        }
        *(u32x4_t*)(Xs(B) + x_lds[k] + e * ROW) = u32x4_t{d[0], d[1], d[2], d[3]};
      }
    }
  };
  auto store_chunk = [&](auto Rc, auto Bc) {
    static_for<NPC>([&](auto Ic) { store_piece(Rc, Bc, Ic); });
  };

  // the load cursor: block-loop index of its unit, next chunk, end of the unit
  int lu = blockIdx.x;
  Unit cu = decode(lu);                     // the compute cursor's unit
  int lc = cu.lo, lhi = cu.hi;
  tile_offsets(cu.pb, cu.m0);
  // Issue the next stream position into register set R.  With two sets a
  // unit's first chunk always goes to set 0: when the stream would put it in
  // set 1 (the previous unit had an odd chunk count) that position is a
  // bubble and the unit start fills set 1 itself.  A position with nothing to load (a
  // bubble, or past the block's last chunk) reloads the cursor's previous
  // chunk into the free set, so that every position issues the same loads
  // and each wait covers exactly one register set.
  bool bubble = false;
  auto issue = [&](auto Rc) {
    constexpr int R = decltype(Rc)::value % NSET;
    bool fresh = true;
    if (lc >= lhi) {
      const int nu = lu + (int)gridDim.x;
      if (R == 0 && nu < units) {
        lu = nu;
        const Unit d = decode(nu);
        lc = d.lo;
        lhi = d.hi;
        tile_offsets(d.pb, d.m0);
      } else {
        fresh = false;
        if (nu < units) bubble = true;
      }
    }
    load_chunk(Rc, (fresh ? lc : lc - 1) * KC);
    if (fresh) ++lc;
  };

  // The k-steps of the chunk in LDS buffer B; with ST, register set B^1 is
  // staged into buffer B^1 at the same time, its LDS stores spread over the
  // k-steps and interleaved with the MFMAs (the matrix core runs while the
  // staging instructions issue).
  auto mfma_chunk = [&](auto Bc, auto STc) {
    constexpr int B = decltype(Bc)::value;
    constexpr bool ST = decltype(STc)::value;
    std::integral_constant<int, B ^ 1> other;
    const char* Xb = Xs(B);
    const char* Ab = As(B);
    u32x4_t pf[3][FP], wf[3][FC];
    auto read_frags = [&](int s, int fb) {
#pragma unroll
      for (int f = 0; f < FP; ++f) pf[fb][f] = *(const u32x4_t*)(Xb + pbase + f * 32 * ROW + s * 32);
#pragma unroll
      for (int f = 0; f < FC; ++f) wf[fb][f] = *(const u32x4_t*)(Ab + wbase + f * 32 * ROW + s * 32);
    };
    read_frags(0, 0);
    if (NS > 1) read_frags(1, 1);
    static_for<NS>([&](auto Sc) {
      constexpr int s = decltype(Sc)::value;
      constexpr bool ahead = s + 2 < NS;
      if constexpr (ahead) read_frags(s + 2, (s + 2) % 3);
      // this step's share of the staging pieces
      constexpr int p0 = ST ? s * NPC / NS : 0, p1 = ST ? (s + 1) * NPC / NS : 0;
      static_for<p1 - p0>([&](auto Jc) {
        store_piece(other, other, std::integral_constant<int, p0 + decltype(Jc)::value>{});
      });
#pragma unroll
      for (int fp = 0; fp < FP; ++fp)
#pragma unroll
        for (int fc = 0; fc < FC; ++fc) mma32(acc[fp][fc], pf[s % 3][fp], wf[s % 3][fc]);
      constexpr int NM = FP * FC, NR = ahead ? FP + FC : 0, NW = p1 - p0;
      constexpr int NMAX = NM > NR ? (NM > NW ? NM : NW) : (NR > NW ? NR : NW);
#pragma unroll
      for (int i = 0; i < NMAX; ++i) {
        if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        if (i < NW) {
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);             // a piece's VALU packing
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);             // its LDS write
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  std::integral_constant<int, 0> s0, b0;
  std::integral_constant<int, 1> s1, b1;
  std::true_type stage;
  std::false_type no_stage;
  issue(s0);
  if constexpr (NSET == 2) issue(s1);
  bool first_unit = true;
  int u = blockIdx.x;
  for (;;) {
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int j = 0; j < FC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    const int n = cu.hi - cu.lo;
    // chunk i of the unit is in register set i % NSET and is read from LDS
    // buffer i & 1; the loop is unrolled by two so that both are known at
    // compile time
    __syncthreads();                 // LDS is free: previous MFMAs and epilogue are done
    if (first_unit) store_bias();
    first_unit = false;
    if (bubble) {                    // chunk 1 was not prefetched
      bubble = false;
      issue(s1);
    }
    store_chunk(s0, b0);
    issue(s0);
    __syncthreads();
    // full iterations only reach the back edge, so that the loads in flight
    // there are always set 1 then set 0 (a partial iteration on the back
    // edge would make the compiler wait for both sets at every store)
    int i = 0;
    for (; i + 2 < n; i += 2) {
      mfma_chunk(b0, stage);         // + chunk i+1: set 1 -> buffer 1 (its last reader passed the previous barrier)
      issue(s1);
      __syncthreads();
      mfma_chunk(b1, stage);         // + chunk i+2: set 0 -> buffer 0
      issue(s0);
      __syncthreads();
    }
    mfma_chunk(b0, no_stage);        // the last one or two chunks
    if (i + 1 < n) {
      store_chunk(s1, b1);
      issue(s1);
      __syncthreads();
      mfma_chunk(b1, no_stage);
    }
    __syncthreads();
    if (S == 1) {
      store_tile<WM, WN, FP, FC, RES>(a, pl, smem, Bv, acc, cu.pb * BN, cu.m0);
    } else {
      f32x4_t* dst = partial_base<FP, FC>(pl.ws, cu.id) + tid;
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
    u += (int)gridDim.x;
    if (u >= units) break;
    cu = decode(u);
  }
}

// Second pass of split-K.  One block per (tile, wave of the first pass):
// its 256 threads split that wave's 64 x FP*FC*4 float4 partial values four
// ways (more loads in flight per CU), add the S slices in slice order, apply
// bias, residual and activation and store straight from the registers (each
// value is four consecutive pixels of one channel).
template <int WM, int WN, int FP, int FC>
__global__ __launch_bounds__(kThreads) void conv1x1_reduce(const ConvArgs a, const PwPlan pl) {
  constexpr int BN = 32 * WN * FP, BM = 32 * WM * FC;
  constexpr int SUBM = 32 * FC, SUBN = 32 * FP;
  constexpr int NV = FP * FC * 4;           // float4 values per lane of the first pass
  constexpr int PER = NV / 4;               // of those, per thread here
  static_assert(NV % 4 == 0, "four threads per lane");
  const int t = blockIdx.x >> 2, w = blockIdx.x & 3;
  const int wm = w / WN, wn = w - (w / WN) * WN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, part = tid >> 6;     // first-pass lane, quarter of its values
  const int l32 = lane & 31, kg = lane >> 5;
  const int pb = t / pl.nmb;
  const int q0 = pb * BN + wn * SUBN, m0 = (t - pb * pl.nmb) * BM + wm * SUBM;
  const int HW = a.H * a.W, M = a.M, Q = a.N * HW;
  // the bias of each value's channel, then every slice's partials
  float bvk[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) bvk[k] = bias_bf16_at(a.bias, M, m0 + (((part * PER + k) >> 2) % FC) * 32 + l32);
  f32x4_t sum[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) sum[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  add_slices<PER>(partial_base<FP, FC>(pl.ws, (int64_t)t * pl.splits) + w * 64 + lane + part * PER * kThreads,
                  kThreads * NV, kThreads, pl.splits, sum);
  const uint16_t* R = (const uint16_t*)a.res;   // residual, added after the bias
  uint16_t* Y = (uint16_t*)a.Y;
  const bool y8 = (((uintptr_t)Y) & 7) == 0;
  with_act(a.act, [&](auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = part * PER + k;             // value index (fp*FC + fc)*4 + g
      const int g = i & 3, fc = (i >> 2) % FC, fp = (i >> 2) / FC;
      const int m = m0 + fc * 32 + l32;
      const int qb = q0 + fp * 32 + 8 * g + 4 * kg;   // the value's first pixel
      if (m >= M || qb >= Q) continue;
      const float bv = bvk[k];
      float v[4] = {sum[k][0] + bv, sum[k][1] + bv, sum[k][2] + bv, sum[k][3] + bv};
      if (R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = qb + j;
          if (q < Q) {
            const int n = q / HW;
            v[j] += bf16_to_f32(R[((int64_t)n * M + m) * HW + (q - n * HW)]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = act_c<ACT>(v[j]);
      // four consecutive pixels of one plane at an 8-byte aligned address
      // go out as one store, any others element by element
      const int n = qb / HW, p = qb - n * HW;
      const int64_t off = ((int64_t)n * M + m) * HW + p;
      if (y8 && qb + 3 < Q && p + 3 < HW && (off & 3) == 0) {
        *(u32x2_t*)(Y + off) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = qb + j;
          if (q < Q) {
            const int nj = q / HW;
            Y[((int64_t)nj * M + m) * HW + (q - nj * HW)] = (uint16_t)(pack_bf16x2(v[j], 0.f) & 0xffffu);
          }
        }
      }
    }
  });
}

template <int WM, int WN, int FP, int KC>
int launch_fp(const ConvArgs& a, const PwPlan& p, hipStream_t s) {
  constexpr int FC = 2;
  dim3 grid(p.grid, 1, 1);
  // the residual epilogue is a separate instantiation, so that the plain
  // kernels keep their registers
  auto go = [&](auto Pc, auto Rc) {
    constexpr int P = decltype(Pc)::value;
    constexpr bool R = decltype(Rc)::value;
    hipLaunchKernelGGL((conv1x1_bf16<WM, WN, FP, FC, KC, P, R>), grid, dim3(kThreads), p.lds, s, a, p);
  };
  auto by_p = [&](auto Rc) {
    switch (p.P) {
      case 4: go(std::integral_constant<int, 4>{}, Rc); break;
      case 2: go(std::integral_constant<int, 2>{}, Rc); break;
      default: go(std::integral_constant<int, 1>{}, Rc); break;
    }
  };
  if (a.res) by_p(std::true_type{});
  else by_p(std::false_type{});
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
