// gemm_conv.hpp -- the problems the MFMA tile engine runs: Gemm / batched
// MatMul, and convolution as a GEMM over (output channel) x (output pixel).
// Each *.hip unit instantiates these for one input type.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "engine.hpp"

namespace ox {

// ------------------------------------------------------------- epilogues --

// Float path: v = alpha*acc + beta*bias[ch]; activation; store as T.
template <typename T>
__device__ __forceinline__ void store_float(T* y, float v);
template <> __device__ __forceinline__ void store_float<float>(float* y, float v) { *y = v; }
template <> __device__ __forceinline__ void store_float<uint16_t>(uint16_t* y, float v) {
  *y = f32_to_bf16(v);
}

// ----------------------------------------------------- Gemm / MatMul kernel --
//
// L = A' (rows = i), R = B' (cols = j).  LK: A stored [M,K]; !LK: [K,M].
// RK: B stored [N,K] (transB); !RK: [K,N].  z = batch index.

// Block -> tile order.  The dispatcher deals a 1-D grid's blocks to the
// eight XCDs in turn (block w to XCD w % 8), and each XCD has an L2 of its
// own: XCD x is given one contiguous run of the tile order, and that order
// walks groups of a.tile_group row tiles column by column, so that the
// tiles an XCD runs together share their A rows and B columns in its L2.
struct TilePos {
  int z, row0, col0;
};
template <int BM, int BN>
__device__ __forceinline__ TilePos gemm_tile_pos(const GemmArgs& a) {
  const int nrt = (a.rows + BM - 1) / BM, nct = (a.cols + BN - 1) / BN;
  const int nb = nrt * nct, total = nb * a.batch;
  const int w = blockIdx.x;
  const int q = total >> 3, rmd = total & 7, x = w & 7, j = w >> 3;
  const int t = x * q + min(x, rmd) + j;
  const int z = t / nb, u = t - z * nb;
  const int g = a.tile_group;
  const int grp = u / (g * nct), in = u - grp * (g * nct);
  const int gr = min(g, nrt - grp * g);
  const int tr = grp * g + in % gr, tc = in / gr;
  return {z, tr * BM, tc * BN};
}

// One block's tile.  int8: rows are activations (x_q [M,K]), columns weight
// channels; FLIP reads uint8 activations in their int8 view, WZ adds the
// weight zero-point term (both chosen per launch from the parameter block).
template <int DT, int BM, int BN, int BKU, int D, bool BUF, bool LK, bool RK, bool FLIP, bool WZ>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, char* smem, const I8View& q) {
  typedef typename Traits<DT>::T T;
  typedef typename Traits<DT>::Acc Acc;

  const TilePos tp = gemm_tile_pos<BM, BN>(a);
  const int z = tp.z, row0 = tp.row0, col0 = tp.col0;
  const T* L = (const T*)a.L + (int64_t)z * a.sl;
  const T* R = (const T*)a.R + (int64_t)z * a.sr;

  Acc acc[BM / 32][BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < BN / 32; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  int ks[WaveTile<DT, BM, BN>::FM] = {};

  if constexpr (BUF) {
    typename std::conditional<LK, LoadRowKB<DT, BM, BKU, FLIP>, LoadColKB<DT, BM, BKU, FLIP>>::type la;
    typename std::conditional<RK, LoadRowKB<DT, BN, BKU>, LoadColKB<DT, BN, BKU>>::type lb;
    la.init(L, a.ldl, row0, a.rows, a.K);
    lb.init(R, a.ldr, col0, a.cols, a.K);
    engine_mainloop<DT, BM, BN, BKU, WZ ? 1 : 0, D>(la, lb, a.K, smem, acc, ks);
  } else {
    typename std::conditional<LK, LoadRowK<DT, BM, BKU, FLIP>, LoadColK<DT, BM, BKU, FLIP>>::type la;
    typename std::conditional<RK, LoadRowK<DT, BN, BKU>, LoadColK<DT, BN, BKU>>::type lb;
    if constexpr (LK) {
      la.init(L, a.ldl, row0, a.rows, a.K, a.l_vec);
    } else {
      const int r = row0 + threadIdx.x % BM;
      la.init_col(L + r, r < a.rows, a.ldl, a.K);
    }
    if constexpr (RK) {
      lb.init(R, a.ldr, col0, a.cols, a.K, a.r_vec);
    } else {
      const int c = col0 + threadIdx.x % BN;
      lb.init_col(R + c, c < a.cols, a.ldr, a.K);
    }
    engine_mainloop<DT, BM, BN, BKU, WZ ? 1 : 0, 1>(la, lb, a.K, smem, acc, ks);
  }

  if constexpr (DT == DT_I8) {
    // weight zero points: acc -= w_zp[ch] * sum_k (x - x_zp) over the row,
    // the row sums completed in LDS (all in wrapping 32-bit arithmetic)
    int* S = (int*)smem;
    if constexpr (WZ) {
      ksums_to_lds<DT, BM, BN, 1>(ks, S);
      __syncthreads();
    }
    // sum_k (x - x_zp) = S - K*x_zp; under FLIP the loader's zeros past K
    // were summed as -128 each
    constexpr int KSTEP = BKU * 4 * Traits<DT>::EPC;
    const int kzx = a.K * q.xzp - (FLIP ? 128 * ((a.K + KSTEP - 1) / KSTEP * KSTEP - a.K) : 0);
    // one column fragment at a time: its parameters are read before its
    // stores (loads behind earlier stores would wait for those stores)
    constexpr int FM = BM / 32, FN = BN / 32;
    constexpr int SMEM = 2 * (BM + BN) * Lds<BKU>::ROWB, SOFF = (BM * 4 + 15) / 16 * 16;
    auto out = [&](auto yk) {
      typedef typename decltype(yk)::type Y_T;
      Y_T* Y = (Y_T*)a.Y + (int64_t)z * a.sy;
      if constexpr (SOFF + stage_rows_bytes<Y_T, BM, BN>() <= SMEM) {
        // through LDS (after the row sums S), whole-row 16-byte stores
        if (rows_vec_ok(Y, a.ldy, a.cols)) {
          if constexpr (!WZ) __syncthreads();   // (WZ: the row sums' barrier did it)
          store_tile_rows<Y_T, BM, BN, SOFF>(Y, a.ldy, row0, col0, a.rows, a.cols, smem, [&](Y_T* E, int EROW) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
              const int c = lane_col<BN>(fn), cc = min(col0 + c, a.cols - 1);
              const int cb = q.bias[cc], cw = WZ ? q.wzp[cc] : 0;
              const double cm = std::is_same<Y_T, int8_t>::value ? q.mult[cc] : 0.0;
              wait_vmem();
#pragma unroll
              for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int r = lane_row<BM>(fm, i);
                  uint32_t u = (uint32_t)acc[fm][fn][i] + (uint32_t)cb;
                  if constexpr (WZ) u -= (uint32_t)cw * (uint32_t)(S[r] - kzx);
                  if constexpr (std::is_same<Y_T, int8_t>::value)
                    E[r * EROW + c] = (int8_t)(requant((int)u, cm, q.yzp) ^ q.ym);
                  else
                    E[r * EROW + c] = (int)u;
                }
            }
          });
          return;
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = col0 + lane_col<BN>(fn), cc = min(col, a.cols - 1);
        const int cb = q.bias[cc], cw = WZ ? q.wzp[cc] : 0;
        const double cm = std::is_same<Y_T, int8_t>::value ? q.mult[cc] : 0.0;
        wait_vmem();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = lane_row<BM>(fm, i), row = row0 + r;
            if (row < a.rows && col < a.cols) {
              uint32_t u = (uint32_t)acc[fm][fn][i] + (uint32_t)cb;
              if constexpr (WZ) u -= (uint32_t)cw * (uint32_t)(S[r] - kzx);
              if constexpr (std::is_same<Y_T, int8_t>::value)
                Y[(int64_t)row * a.ldy + col] = (int8_t)(requant((int)u, cm, q.yzp) ^ q.ym);
              else
                Y[(int64_t)row * a.ldy + col] = (int)u;
            }
          }
      }
    };
    if (a.out_dt == DT_I32) out(std::common_type<int32_t>{});
    else out(std::common_type<int8_t>{});
  } else {
    T* Y = (T*)a.Y + (int64_t)z * a.sy;
    const T* bias = (const T*)a.bias;
    // beta * bias of this lane's columns, read before any store
    constexpr int FN = BN / 32;
    float bc[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      bc[fn] = bias ? a.beta * to_f32(bias[min(col0 + lane_col<BN>(fn), a.cols - 1)]) : 0.0f;
    wait_vmem();
    constexpr int SMEM = 2 * (BM + BN) * Lds<BKU>::ROWB;
    if constexpr (stage_rows_bytes<T, BM, BN>() <= SMEM) {
      // through LDS, whole-row 16-byte stores
      if (rows_vec_ok(Y, a.ldy, a.cols)) {
        __syncthreads();
        with_act(a.act, [&](auto act_k) {
          constexpr int ACT = decltype(act_k)::value;
          store_tile_rows<T, BM, BN, 0>(Y, a.ldy, row0, col0, a.rows, a.cols, smem, [&](T* E, int EROW) {
            for_each_result_fn<BM, BN>(acc, [&](int fn, int r, int c, float v) {
              float o = a.alpha * v;
              if (bias) o += bc[fn];
              store_float(E + r * EROW + c, act_c<ACT>(o));
            });
          });
        });
        return;
      }
    }
    with_act(a.act, [&](auto act_k) {
      constexpr int ACT = decltype(act_k)::value;
      for_each_result_fn<BM, BN>(acc, [&](int fn, int r, int c, float v) {
        const int row = row0 + r, col = col0 + c;
        if (row < a.rows && col < a.cols) {
          float o = a.alpha * v;
          if (bias) o += bc[fn];
          store_float(Y + (int64_t)row * a.ldy + col, act_c<ACT>(o));
        }
      });
    });
  }
}

template <int DT, int BM, int BN, int BKU, int D, bool BUF, bool LK, bool RK>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * Lds<BKU>::ROWB];
  I8View q;
  if constexpr (DT == DT_I8) {
    q.init(a.i8);
    // uniform per launch: one of four instantiations runs
    if (q.xm) {
      if (q.wz) gemm_tile<DT, BM, BN, BKU, D, BUF, LK, RK, true, true>(a, smem, q);
      else gemm_tile<DT, BM, BN, BKU, D, BUF, LK, RK, true, false>(a, smem, q);
    } else {
      if (q.wz) gemm_tile<DT, BM, BN, BKU, D, BUF, LK, RK, false, true>(a, smem, q);
      else gemm_tile<DT, BM, BN, BKU, D, BUF, LK, RK, false, false>(a, smem, q);
    }
  } else {
    gemm_tile<DT, BM, BN, BKU, D, BUF, LK, RK, false, false>(a, smem, q);
  }
}

// Row tiles per group of the tile order: an XCD's share of the tiles as a
// g x c block of tiles whose A rows (g*BM) and B columns (c*BN) are about
// equal in number (the least operand data for that many tiles).
// OX_GEMM_GROUP pins g (measurements).
template <int BM, int BN>
int gemm_tile_group(int64_t nrt, int64_t total) {
  int64_t g = (int64_t)(std::sqrt((double)((total + 7) / 8) * BN / BM) + 0.5);
  if (const char* e = getenv("OX_GEMM_GROUP")) g = atoi(e);
  return (int)std::max<int64_t>(1, std::min(g, nrt));
}

template <int DT, int BM, int BN, int BKU, int D, bool BUF>
int launch_gemm_tile_k(const GemmArgs& a0, hipStream_t s) {
  const int64_t nrt = (a0.rows + BM - 1) / BM, nct = (a0.cols + BN - 1) / BN;
  const int64_t total = nrt * nct * a0.batch;
  if (total >= ((int64_t)1 << 31)) return (int)hipErrorInvalidConfiguration;
  GemmArgs a = a0;
  a.tile_group = gemm_tile_group<BM, BN>(nrt, total);
  dim3 grid((unsigned)total);
  if constexpr (DT == DT_I8) {
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BKU, D, BUF, true, true>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.l_kmajor && a.r_kmajor)
      hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BKU, D, BUF, true, true>), grid, dim3(kThreads), 0, s, a);
    else if constexpr (BUF && DT != DT_F32)
      return (int)hipErrorInvalidValue;   // K-strided narrow operands never take BUF
    else if (a.l_kmajor)
      hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BKU, D, BUF, true, false>), grid, dim3(kThreads), 0, s, a);
    else if (a.r_kmajor)
      hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BKU, D, BUF, false, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BKU, D, BUF, false, false>), grid, dim3(kThreads), 0, s, a);
  }
  return (int)hipGetLastError();
}

// With few output tiles (at most two blocks per CU) one block runs the whole
// K loop and every K stage costs about one global-load latency: a long K (16
// stages or more of 64 bytes per row; 4 or more when the grid has at most 64
// blocks) then takes four 64-byte units per stage, a quarter of the stages
// (small tiles only: the LDS of the deeper stages would cost a larger grid
// its occupancy).
template <int DT, int BM, int BN>
constexpr bool deep_k_tile() { return BM <= 64 && BN <= 64; }
template <int DT>
bool deep_k(int64_t K, int64_t blocks) {
  constexpr int KSTEP1 = 4 * Traits<DT>::EPC;
  const int64_t stages = (K + KSTEP1 - 1) / KSTEP1;
  // (a grid of at most 64 blocks leaves most CUs idle: there even 4 stages)
  return (blocks <= 512 && stages >= 16) || (blocks <= 64 && stages >= 4);
}

// Stage shape of a launch, BKU x D (K units per stage x stages in flight):
// two units per stage with two stages in flight for tiles up to 64 x 128
// once K has 8 units or more (the loads of four units stay in flight across
// the MMAs), 1 x 1 otherwise (128 x 128 would lose an occupancy level to the
// registers of a second stage).  Measured, bf16 (us): 1000x4096x1024 on
// 64x128 28.1 / 30.2 / 21.3 for 1x1 / 4x1 / 2x2; 1000x1024x4096 on 32x64
// 59.8 / 29.1 / 26.8; 256x4096x1024 on 32x64 18.7 / 10.8 / 10.4.
// OX_GEMM_STAGES ("1x1", "4x1", "2x2") pins one for any tile (measurements).
template <int DT, int BM, int BN>
int gemm_stages(const GemmArgs& a) {
  if (const char* e = getenv("OX_GEMM_STAGES")) {
    static const char* names[] = {"1x1", "4x1", "2x2"};
    for (int i = 0; i < 3; ++i)
      if (!strcmp(e, names[i])) return i;
  }
  constexpr int KSTEP1 = 4 * Traits<DT>::EPC;
  if (BM * BN <= 64 * 128 && (a.K + KSTEP1 - 1) / KSTEP1 >= 8) return 2;
  return 0;
}

// Whether the branch-free buffer loaders apply: a K-contiguous operand needs
// 16-byte aligned rows and K a multiple of 16 bytes; a K-strided one fp32
// elements (narrower ones would be widened in registers that are still
// loading); every byte offset a block forms from its base stays below 2^31.
template <int DT, int BM, int BN>
bool gemm_buf_ok(const GemmArgs& a) {
  const int64_t es = sizeof(typename Traits<DT>::T), lim = (int64_t)1 << 31;
  const int64_t kb = (int64_t)a.K * es;
  auto side = [&](bool kmajor, int vec, int64_t ld, int tile) {
    return kmajor ? vec && kb % 16 == 0 && tile * ld * es + kb < lim
                  : es == 4 && kb * ld + tile * es < lim;
  };
  return side(DT == DT_I8 || a.l_kmajor, a.l_vec, a.ldl, BM) &&
         side(DT == DT_I8 || a.r_kmajor, a.r_vec, a.ldr, BN);
}

template <int DT, int BM, int BN>
int launch_gemm_tile(const GemmArgs& a, hipStream_t s) {
  const int st = gemm_stages<DT, BM, BN>(a);
  if (!gemm_buf_ok<DT, BM, BN>(a)) {
    // the gathering loaders, one stage in flight: four units per stage for
    // the small tiles with a long K
    bool deep = false;
    if constexpr (deep_k_tile<DT, BM, BN>()) {
      const int64_t blocks = (int64_t)((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM) * a.batch;
      deep = deep_k<DT>(a.K, blocks);
    }
    return deep || st == 1 ? launch_gemm_tile_k<DT, BM, BN, 4, 1, false>(a, s)
                           : launch_gemm_tile_k<DT, BM, BN, 1, 1, false>(a, s);
  }
  switch (st) {
    case 1: return launch_gemm_tile_k<DT, BM, BN, 4, 1, true>(a, s);
    case 2: return launch_gemm_tile_k<DT, BM, BN, 2, 2, true>(a, s);
    default: return launch_gemm_tile_k<DT, BM, BN, 1, 1, true>(a, s);
  }
}

// ---------------------------------------------------- split-K float Gemm --
//
// A Gemm with too few output tiles to fill the chip and a long K: slice z of
// the grid takes K range [z*kslice, (z+1)*kslice) (a multiple of the deep
// stage, so vector alignment is kept) and writes its fp32 partial tile to
// ws[z][rows][cols]; a second kernel adds the slices in order and applies
// alpha, beta*bias and the activation.  32x64 tiles (the tile a problem
// this small is given), four K units per stage.

template <int DT, bool LK, bool RK, bool BUF>
__global__ __launch_bounds__(kThreads) void gemm_splitk_kernel(const GemmArgs a, int kslice,
                                                               float* ws) {
  typedef typename Traits<DT>::T T;
  // buffer loaders: two units x two stages in flight; else four units, one
  constexpr int BM = 32, BN = 64, BKU = BUF ? 2 : 4, D = BUF ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * Lds<BKU>::ROWB];
  const int z = blockIdx.z, row0 = blockIdx.y * BM, col0 = blockIdx.x * BN;
  const int k0 = z * kslice;
  const int Kz = min(kslice, a.K - k0);          // >= 1: the host makes every slice non-empty
  const T* L = (const T*)a.L + (LK ? (int64_t)k0 : (int64_t)k0 * a.ldl);
  const T* R = (const T*)a.R + (RK ? (int64_t)k0 : (int64_t)k0 * a.ldr);
  f32x4_t acc[BM / 32][BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < BN / 32; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (BUF) {
    typename std::conditional<LK, LoadRowKB<DT, BM, BKU>, LoadColKB<DT, BM, BKU>>::type la;
    typename std::conditional<RK, LoadRowKB<DT, BN, BKU>, LoadColKB<DT, BN, BKU>>::type lb;
    la.init(L, a.ldl, row0, a.rows, Kz);
    lb.init(R, a.ldr, col0, a.cols, Kz);
    engine_mainloop<DT, BM, BN, BKU, 0, D>(la, lb, Kz, smem, acc);
  } else {
    typename std::conditional<LK, LoadRowK<DT, BM, BKU>, LoadColK<DT, BM, BKU>>::type la;
    typename std::conditional<RK, LoadRowK<DT, BN, BKU>, LoadColK<DT, BN, BKU>>::type lb;
    if constexpr (LK) {
      la.init(L, a.ldl, row0, a.rows, Kz, a.l_vec);
    } else {
      const int r = row0 + threadIdx.x % BM;
      la.init_col(L + r, r < a.rows, a.ldl, Kz);
    }
    if constexpr (RK) {
      lb.init(R, a.ldr, col0, a.cols, Kz, a.r_vec);
    } else {
      const int c = col0 + threadIdx.x % BN;
      lb.init_col(R + c, c < a.cols, a.ldr, Kz);
    }
    engine_mainloop<DT, BM, BN, BKU>(la, lb, Kz, smem, acc);
  }
  float* P = ws + (int64_t)z * a.rows * a.cols;
  for_each_result<BM, BN>(acc, [&](int r, int c, float v) {
    const int row = row0 + r, col = col0 + c;
    if (row < a.rows && col < a.cols) P[(int64_t)row * a.cols + col] = v;
  });
}

template <int DT, int ACT>
__global__ __launch_bounds__(kThreads) void gemm_splitk_reduce(const GemmArgs a, int S,
                                                               const float* ws) {
  typedef typename Traits<DT>::T T;
  const int64_t total = (int64_t)a.rows * a.cols;
  const T* bias = (const T*)a.bias;
  T* Y = (T*)a.Y;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    float v = 0.0f;
    for (int z = 0; z < S; ++z) v += ws[(int64_t)z * total + i];
    const int row = (int)(i / a.cols), col = (int)(i - (int64_t)row * a.cols);
    float o = a.alpha * v;
    if (bias) o += a.beta * to_f32(bias[col]);
    store_float(Y + (int64_t)row * a.ldy + col, act_c<ACT>(o));
  }
}

template <int DT>
int launch_gemm_splitk_dt(const GemmArgs& a, int S, int kslice, float* ws, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  dim3 grid((a.cols + 63) / 64, (a.rows + 31) / 32, S);
  // (the slices' bases move by a multiple of four units: the buffer
  // loaders' alignment and offset conditions hold for every slice)
  if (gemm_buf_ok<DT, 32, 64>(a)) {
    if (a.l_kmajor && a.r_kmajor)
      hipLaunchKernelGGL((gemm_splitk_kernel<DT, true, true, true>), grid, dim3(kThreads), 0, s, a, kslice, ws);
    else if constexpr (DT == DT_F32) {
      if (a.l_kmajor)
        hipLaunchKernelGGL((gemm_splitk_kernel<DT, true, false, true>), grid, dim3(kThreads), 0, s, a, kslice, ws);
      else if (a.r_kmajor)
        hipLaunchKernelGGL((gemm_splitk_kernel<DT, false, true, true>), grid, dim3(kThreads), 0, s, a, kslice, ws);
      else
        hipLaunchKernelGGL((gemm_splitk_kernel<DT, false, false, true>), grid, dim3(kThreads), 0, s, a, kslice, ws);
    }
  } else if (a.l_kmajor && a.r_kmajor)
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, true, true, false>), grid, dim3(kThreads), 0, s, a, kslice, ws);
  else if (a.l_kmajor)
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, true, false, false>), grid, dim3(kThreads), 0, s, a, kslice, ws);
  else if (a.r_kmajor)
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, false, true, false>), grid, dim3(kThreads), 0, s, a, kslice, ws);
  else
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, false, false, false>), grid, dim3(kThreads), 0, s, a, kslice, ws);
  const int64_t total = (int64_t)a.rows * a.cols;
  const int nb = (int)std::min<int64_t>(2048, (total + kThreads - 1) / kThreads);
  const float* wsc = ws;
  switch (a.act) {
    case ACT_RELU:
      hipLaunchKernelGGL((gemm_splitk_reduce<DT, ACT_RELU>), dim3(nb), dim3(kThreads), 0, s, a, S, wsc);
      break;
    case ACT_RELU6:
      hipLaunchKernelGGL((gemm_splitk_reduce<DT, ACT_RELU6>), dim3(nb), dim3(kThreads), 0, s, a, S, wsc);
      break;
    case ACT_GELU:
      hipLaunchKernelGGL((gemm_splitk_reduce<DT, ACT_GELU>), dim3(nb), dim3(kThreads), 0, s, a, S, wsc);
      break;
    default:
      hipLaunchKernelGGL((gemm_splitk_reduce<DT, ACT_NONE>), dim3(nb), dim3(kThreads), 0, s, a, S, wsc);
      break;
  }
  return (int)hipGetLastError();
}

template <int DT>
int launch_gemm_dt(const GemmArgs& a, int tile, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (tile) {
    case TILE_128x128: return launch_gemm_tile<DT, 128, 128>(a, s);
    case TILE_64x128: return launch_gemm_tile<DT, 64, 128>(a, s);
    case TILE_128x64: return launch_gemm_tile<DT, 128, 64>(a, s);
    case TILE_64x64: return launch_gemm_tile<DT, 64, 64>(a, s);
    case TILE_32x64: return launch_gemm_tile<DT, 32, 64>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ conv kernel --
//
// rows = output channels of group z (L = weights [M/g, K], K contiguous),
// cols = output pixels over the batch, n = (img*Ho + oh)*Wo + ow.
// KIND 0: implicit GEMM (im2col gathered on the fly); KIND 1: 1x1, stride 1,
// no pad, where column n of image img is X[img, c, p] with p = n % (H*W);
// KIND 2: the same 1x1 through the branch-free buffer loaders with D stages
// in flight (fp32 columns one by one, bf16 in pixel pairs, int8 in groups of
// four; operands whose byte offsets stay below 2^31); KIND 3: the fp32
// implicit GEMM through them.

template <int DT, int BM, int BN, int BKU, int KIND, bool FLIP, bool WZ, int D = 1>
__device__ __forceinline__ void conv_tile(const ConvArgs& a, char* smem, const I8View& q) {
  typedef typename Traits<DT>::T T;
  typedef typename Traits<DT>::Acc Acc;

  const int g = blockIdx.z, row0 = blockIdx.y * BM, col0 = blockIdx.x * BN;
  const int Mpg = a.M / a.group, cpg = a.C / a.group;
  const int KK = a.kH * a.kW, K = cpg * KK;
  const int HoWo = a.Ho * a.Wo, HW = a.H * a.W, NP = a.N * HoWo;

  Acc acc[BM / 32][BN / 32];
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
#pragma unroll
    for (int j = 0; j < BN / 32; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  int ks[WaveTile<DT, BM, BN>::FN] = {};

  if constexpr (KIND == 3) {
    // fp32 implicit GEMM through the buffer loaders
    LoadRowKB<DT, BM, BKU> la;
    la.init((const T*)a.Wt + (int64_t)g * Mpg * K, K, row0, Mpg, K);
    LoadIm2colB<BN, BKU> lb;
    const int n = col0 + threadIdx.x % BN;
    const bool nvalid = n < NP;
    const int img = nvalid ? n / HoWo : 0;
    const int p = nvalid ? n - img * HoWo : 0;
    const int oh = p / a.Wo, ow = p - (p / a.Wo) * a.Wo;
    lb.rs = operand_rsrc(a.X);
    lb.vimg = (uint32_t)(((int64_t)img * a.C + (int64_t)g * cpg) * HW * 4);
    lb.ih0 = oh * a.sh - a.pt;
    lb.iw0 = ow * a.sw - a.pl;
    lb.valid = nvalid;
    lb.H = a.H;
    lb.W = a.W;
    lb.HW = HW;
    lb.kH = a.kH;
    lb.kW = a.kW;
    lb.KK = KK;
    lb.dh = a.dh;
    lb.dw = a.dw;
    lb.K = K;
    engine_mainloop<DT, BM, BN, BKU, 0, D>(la, lb, K, smem, acc, ks);
  } else if constexpr (KIND == 2) {
    LoadRowKB<DT, BM, BKU> la;
    la.init((const T*)a.Wt + (int64_t)g * Mpg * K, K, row0, Mpg, K);
    // this thread's column (fp32; bf16 on an odd plane), pair of columns
    // (bf16) or group of four columns (int8)
    auto run = [&](auto lbk, auto cgk) {
      typedef typename decltype(lbk)::type LB;
      constexpr int CG = decltype(cgk)::value;
      const int n = col0 + CG * (threadIdx.x % (BN / CG));
      const bool nvalid = n < NP;
      const int img = nvalid ? n / HoWo : 0;
      const uint32_t off = (uint32_t)((((int64_t)img * a.C + (int64_t)g * cpg) * HW + (n - img * HoWo)) *
                                      (int64_t)sizeof(T));
      LB lb;
      lb.init_off((const T*)a.X, nvalid ? off : 0u, nvalid, HW, K);
      engine_mainloop<DT, BM, BN, BKU, WZ ? 2 : 0, D>(la, lb, K, smem, acc, ks);
    };
    if constexpr (DT == DT_I8) {
      run(std::common_type<LoadColK4B<BN, BKU, FLIP>>{}, std::integral_constant<int, 4>{});
    } else if constexpr (DT == DT_BF16) {
      if (HW % 2 == 0) run(std::common_type<LoadColK2B<BN, BKU>>{}, std::integral_constant<int, 2>{});
      else run(std::common_type<LoadColK1B<BN, BKU>>{}, std::integral_constant<int, 1>{});
    } else {
      run(std::common_type<LoadColKB<DT, BN, BKU, FLIP>>{}, std::integral_constant<int, 1>{});
    }
  } else {
  LoadRowK<DT, BM, BKU> la;
  la.init((const T*)a.Wt + (int64_t)g * Mpg * K, K, row0, Mpg, K, a.w_vec);

  const int n = col0 + threadIdx.x % BN;
  const bool nvalid = n < NP;
  const int img = nvalid ? n / HoWo : 0;
  const int p = nvalid ? n - img * HoWo : 0;
  const T* xg = (const T*)a.X + ((int64_t)img * a.C + (int64_t)g * cpg) * HW;

  typename std::conditional<KIND == 1, LoadColK<DT, BN, BKU, FLIP>, LoadIm2col<DT, BN, BKU, FLIP>>::type lb;
  if constexpr (KIND == 1) {
    lb.init_col(xg + p, nvalid, HW, K);
  } else {
    const int oh = p / a.Wo, ow = p - (p / a.Wo) * a.Wo;
    lb.xb = xg;
    lb.ih0 = oh * a.sh - a.pt;
    lb.iw0 = ow * a.sw - a.pl;
    lb.valid = nvalid;
    lb.H = a.H;
    lb.W = a.W;
    lb.HW = HW;
    lb.kH = a.kH;
    lb.kW = a.kW;
    lb.KK = KK;
    lb.dh = a.dh;
    lb.dw = a.dw;
    lb.K = K;
    // (int8: the padding holds x_zp in the int8 view; under FLIP it is
    // stored as the uint8 byte, flipped with the loaded data)
    if constexpr (DT == DT_I8) lb.pad = (T)(int8_t)(FLIP ? (q.xzp ^ 0x80) : q.xzp);
    else lb.pad = (T)0;
  }

  engine_mainloop<DT, BM, BN, BKU, WZ ? 2 : 0>(la, lb, K, smem, acc, ks);
  }

  constexpr int FM = BM / 32, FN = BN / 32;
  // Y[img, m, p] of output pixel col = img*HoWo + p sits at cb + m*HoWo,
  // cb = img*M*HoWo + p: one base per lane column (clamped into range)
  int64_t cbase[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int col = min(col0 + lane_col<BN>(fn), NP - 1);
    const int im = col / HoWo;
    cbase[fn] = (int64_t)im * a.M * HoWo + (col - im * HoWo);
  }
  auto out_index = [&](int m, int fn) -> int64_t { return cbase[fn] + (int64_t)m * HoWo; };
  if constexpr (DT == DT_I8) {
    // weight zero points: acc -= w_zp[m] * sum over the pixel's taps of
    // (x - x_zp) (padding taps hold x_zp: zero), the column sums completed in
    // LDS (all in wrapping 32-bit arithmetic)
    int* S = (int*)smem;
    if constexpr (WZ) {
      ksums_to_lds<DT, BM, BN, 2>(ks, S);
      __syncthreads();
    }
    // sum over taps of (x - x_zp) = S - K*x_zp (padding taps hold x_zp);
    // under FLIP the loader's zeros past K were summed as -128 each
    constexpr int KSTEP = BKU * 4 * Traits<DT>::EPC;
    const int kzx = K * q.xzp - (FLIP ? 128 * ((K + KSTEP - 1) / KSTEP * KSTEP - K) : 0);
    // one row fragment at a time: its four channels' parameters are read
    // before its stores (loads behind earlier stores would wait for them)
    const bool i32 = a.out_dt == DT_I32;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      int rb[4], rw[4];
      double rm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = g * Mpg + min(row0 + lane_row<BM>(fm, i), Mpg - 1);
        rb[i] = q.bias[m];
        rw[i] = WZ ? q.wzp[m] : 0;
        rm[i] = q.mult[m];
      }
      wait_vmem();
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ml = row0 + lane_row<BM>(fm, i), c = lane_col<BN>(fn), col = col0 + c;
          if (ml < Mpg && col < NP) {
            uint32_t u = (uint32_t)acc[fm][fn][i] + (uint32_t)rb[i];
            if constexpr (WZ) u -= (uint32_t)rw[i] * (uint32_t)(S[c] - kzx);
            const int64_t o = out_index(g * Mpg + ml, fn);
            if (i32) ((int32_t*)a.Y)[o] = (int)u;
            else ((int8_t*)a.Y)[o] = (int8_t)(requant((int)u, rm[i], q.yzp) ^ q.ym);
          }
        }
    }
  } else {
    T* Y = (T*)a.Y;
    const T* bias = (const T*)a.bias;
    const T* R = (const T*)a.res;     // residual, added after the bias (may be Y itself)
    // (A residual, rare on this kernel, is read element by element before
    // each store: R may be Y, and hoisting more of its loads costs the
    // kernel its occupancy in registers.)
    // bf16 without a residual, HoWo even and Y 4-byte aligned: lanes l and
    // l^1 hold the same four channels at two adjacent pixels, so one
    // exchange (DPP quad_perm 1,0,3,2) per two values gives each lane a pixel
    // pair of two of the channels, and every store writes 4 bytes (half the
    // store instructions of element stores).  A pair never straddles two
    // images (HoWo even), and it is inside the tile's columns whenever its
    // first pixel is (NP even).
    const bool pairs = DT == DT_BF16 && (HoWo & 1) == 0 && (((uintptr_t)Y) & 3) == 0;
    auto body = [&](auto with_res) {
      constexpr bool RES = decltype(with_res)::value;
      // The biases of a row fragment are read before its stores (a wait
      // for a load issued after stores waits for those stores too): every
      // fragment's before the first store on tiles of up to two row
      // fragments; one fragment at a time on 128-row tiles, whose registers
      // would otherwise cost a block per CU.
      constexpr bool PRE = FM <= 2;
      float rball[PRE ? FM : 1][4];
      auto load_rb = [&](float (&rb)[4], int fm) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          rb[i] = bias ? to_f32(bias[g * Mpg + min(row0 + lane_row<BM>(fm, i), Mpg - 1)]) : 0.0f;
      };
      if constexpr (PRE) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) load_rb(rball[fm], fm);
        if constexpr (!RES) wait_vmem();
      }
      with_act(a.act, [&](auto act_k) {
        constexpr int ACT = decltype(act_k)::value;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if constexpr (!PRE) {
            load_rb(rball[0], fm);
            if constexpr (!RES) wait_vmem();
          }
          const float* rb = rball[PRE ? fm : 0];
          if constexpr (DT == DT_BF16 && !RES) {
            if (pairs) {
              const bool odd = threadIdx.x & 1;
#pragma unroll
              for (int fn = 0; fn < FN; ++fn) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  o[i] = acc[fm][fn][i];
                  if (bias) o[i] += rb[i];
                  o[i] = act_c<ACT>(o[i]);
                }
                // the even lane keeps channels 0, 1 of its four, the odd
                // lane channels 2, 3; each sends the partner the other two
                auto xchg = [](float v) {
                  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
                };
                const float r0 = xchg(odd ? o[0] : o[2]), r1 = xchg(odd ? o[1] : o[3]);
                const int ce = col0 + (lane_col<BN>(fn) & ~1);
                const int ma = row0 + lane_row<BM>(fm, odd ? 2 : 0);
                const int64_t base = cbase[fn] - (odd ? 1 : 0);
                if (ce < NP) {
                  if (ma < Mpg)
                    *(uint32_t*)(Y + base + (int64_t)(g * Mpg + ma) * HoWo) =
                        odd ? pack_bf16x2(r0, o[2]) : pack_bf16x2(o[0], r0);
                  if (ma + 1 < Mpg)
                    *(uint32_t*)(Y + base + (int64_t)(g * Mpg + ma + 1) * HoWo) =
                        odd ? pack_bf16x2(r1, o[3]) : pack_bf16x2(o[1], r1);
                }
              }
              continue;
            }
          }
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ml = row0 + lane_row<BM>(fm, i), col = col0 + lane_col<BN>(fn);
              if (ml < Mpg && col < NP) {
                const int64_t o_idx = out_index(g * Mpg + ml, fn);
                float o = acc[fm][fn][i];
                if (bias) o += rb[i];
                if constexpr (RES) o += to_f32(R[o_idx]);
                store_float(Y + o_idx, act_c<ACT>(o));
              }
            }
          }
        }
      });
    };
    if (R) body(std::true_type{});
    else body(std::false_type{});
  }
}

template <int DT, int BM, int BN, int BKU, int KIND, int D = 1>
__global__ __launch_bounds__(kThreads) void conv_kernel(const ConvArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * Lds<BKU>::ROWB];
  I8View q;
  if constexpr (DT == DT_I8) {
    q.init(a.i8);
    // uniform per launch: one of four instantiations runs
    if (q.xm) {
      if (q.wz) conv_tile<DT, BM, BN, BKU, KIND, true, true, D>(a, smem, q);
      else conv_tile<DT, BM, BN, BKU, KIND, true, false, D>(a, smem, q);
    } else {
      if (q.wz) conv_tile<DT, BM, BN, BKU, KIND, false, true, D>(a, smem, q);
      else conv_tile<DT, BM, BN, BKU, KIND, false, false, D>(a, smem, q);
    }
  } else {
    conv_tile<DT, BM, BN, BKU, KIND, false, false, D>(a, smem, q);
  }
}

template <int DT, int BM, int BN, int BKU, int D = 1>
int launch_conv_tile_k(const ConvArgs& a, int kind, hipStream_t s) {
  const int Mpg = a.M / a.group;
  const int64_t NP = (int64_t)a.N * a.Ho * a.Wo;
  dim3 grid((unsigned)((NP + BN - 1) / BN), (Mpg + BM - 1) / BM, a.group);
  if constexpr (D > 1) {
    if constexpr (DT == DT_F32)
      if (kind == 3) {
        hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 3, D>), grid, dim3(kThreads), 0, s, a);
        return (int)hipGetLastError();
      }
    hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 2, D>), grid, dim3(kThreads), 0, s, a);
  } else {
    if constexpr (DT == DT_F32)
      if (kind == 3) {
        hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 3>), grid, dim3(kThreads), 0, s, a);
        return (int)hipGetLastError();
      }
    if (kind == 2)
      hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 2>), grid, dim3(kThreads), 0, s, a);
    else if (kind == 1)
      hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 1>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((conv_kernel<DT, BM, BN, BKU, 0>), grid, dim3(kThreads), 0, s, a);
  }
  return (int)hipGetLastError();
}

// Whether a 1x1 convolution takes the buffer loaders (KIND 2): fp32; bf16
// (pixel pairs on even planes with a 4-byte aligned X, single pixels
// otherwise); int8 with planes of whole 4-byte groups and a 4-byte aligned X;
// weight rows of whole 16-byte vectors; X below 2^31 bytes.  OX_CONV_PIPE=0
// turns it off (measurements).
template <int DT>
bool conv_buf_ok(const ConvArgs& a) {
  constexpr int ES = DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1;
  if (!a.w_vec) return false;
  if (DT == DT_BF16 && (a.H * a.W) % 2 == 0 && ((uintptr_t)a.X) % 4 != 0) return false;
  if (DT == DT_I8 && ((a.H * a.W) % 4 != 0 || ((uintptr_t)a.X) % 4 != 0)) return false;
  if (const char* e = getenv("OX_CONV_PIPE"))
    if (!strcmp(e, "0")) return false;
  return (int64_t)a.N * a.C * a.H * a.W * ES < ((int64_t)1 << 31);
}

template <int DT, int BM, int BN>
int launch_conv_tile(const ConvArgs& a, int kind, hipStream_t s) {
  const int64_t NP = (int64_t)a.N * a.Ho * a.Wo;
  const int64_t blocks = ((NP + BN - 1) / BN) * ((a.M / a.group + BM - 1) / BM) * a.group;
  const int64_t K = (int64_t)(a.C / a.group) * a.kH * a.kW;
  bool deep = false;
  if constexpr (deep_k_tile<DT, BM, BN>()) deep = deep_k<DT>(K, blocks);
  // fp32 implicit GEMM through the buffer loaders (KIND 3): weight rows of
  // whole 16-byte vectors, X below 2^31 bytes
  const bool im2col_buf = DT == DT_F32 && kind == 0 && a.w_vec &&
                          (int64_t)a.N * a.C * a.H * a.W * 4 < ((int64_t)1 << 31) &&
                          !(getenv("OX_CONV_PIPE") && !strcmp(getenv("OX_CONV_PIPE"), "0"));
  if ((kind == 1 && conv_buf_ok<DT>(a)) || im2col_buf) {
    const int bk = im2col_buf ? 3 : 2;
    // 4 x 1 where the small tiles go deep (the int8 conformer pointwise
    // conv: 16.3 us against 17.8 us with 2 x 2), else the Gemm's shapes:
    // 2 x 2 for tiles up to 64 x 128 with 8 or more K units, 1 x 1 otherwise
    // (OX_GEMM_STAGES pins one)
    GemmArgs ga;
    memset(&ga, 0, sizeof(ga));
    ga.K = (int)K;
    int st = gemm_stages<DT, BM, BN>(ga);
    if (deep && !getenv("OX_GEMM_STAGES")) st = 1;
    if (st == 1) {
      if constexpr (deep_k_tile<DT, BM, BN>()) return launch_conv_tile_k<DT, BM, BN, 4>(a, bk, s);
    } else if (st == 2) {
      if constexpr (BM * BN <= 64 * 128) return launch_conv_tile_k<DT, BM, BN, 2, 2>(a, bk, s);
    }
    return launch_conv_tile_k<DT, BM, BN, 1>(a, bk, s);
  }
  if constexpr (deep_k_tile<DT, BM, BN>())
    if (deep) return launch_conv_tile_k<DT, BM, BN, 4>(a, kind, s);
  return launch_conv_tile_k<DT, BM, BN, 1>(a, kind, s);
}

template <int DT>
int launch_conv_dt(const ConvArgs& a, int kind, int tile, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (tile) {
    case TILE_128x128: return launch_conv_tile<DT, 128, 128>(a, kind, s);
    case TILE_64x128: return launch_conv_tile<DT, 64, 128>(a, kind, s);
    case TILE_128x64: return launch_conv_tile<DT, 128, 64>(a, kind, s);
    case TILE_64x64: return launch_conv_tile<DT, 64, 64>(a, kind, s);
    case TILE_32x64: return launch_conv_tile<DT, 32, 64>(a, kind, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace ox
