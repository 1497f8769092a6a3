// k_depthwise.hip -- depthwise convolution (group == C == M), VALU only.
//
// The DepthwiseConv choice of "OxiONNX 0.1.7 Released" (Technical Deep Dive,
// item 2): per channel c, Y[n,c] = act(b[c] + sum_{kh,kw} W[c,kh,kw] *
// X[n,c, oh*sh-pt+kh*dh, ow*sw-pl+kw*dw]).  At one or two flops per byte it is
// bound by HBM, so it gets no MFMA: the design goal is to read X once and
// write Y once at full bandwidth.
//
// A block owns P consecutive (n,c) planes (contiguous in NCHW) and a band of
// TH output rows.  It stages the input band of each plane in LDS with its
// halo already materialised (padding cells hold 0, or x_zp for int8), so the
// inner loop has no bounds checks.  The band is copied with 16-byte loads
// where rows are 16-byte aligned.  Each thread then computes a strip of 4
// adjacent outputs of one row, reusing one window of LDS values per kernel
// row across the 4 outputs.  Common shapes (3x3 stride 1/2, 1x9 stride 1,
// dilation 1) are compiled with fixed loop bounds; any other geometry runs a
// generic variant of the same scheme.
#include <algorithm>
#include <cstdlib>

#include "engine.hpp"

namespace ox {

namespace {

template <int DT> struct Dw;
template <> struct Dw<DT_F32> { typedef float T; typedef float A; };
template <> struct Dw<DT_BF16> { typedef uint16_t T; typedef float A; };
template <> struct Dw<DT_I8> { typedef int8_t T; typedef int A; };

template <typename T, typename A> __device__ __forceinline__ A widen(T v);
template <> __device__ __forceinline__ float widen<float, float>(float v) { return v; }
template <> __device__ __forceinline__ float widen<uint16_t, float>(uint16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ int widen<int8_t, int>(int8_t v) { return (int)v; }

struct DwPlan {
  int TH;     // output rows per block
  int P;      // planes per block
  int RIN;    // input rows staged per plane
  int WP;     // staged row width (input columns incl. left/right halo)
  int OWT;    // outputs per thread strip (4)
  FastDiv fd_w;       // input row length W
  FastDiv fd_plane;   // H*W: span of one input plane (blocks of several planes)
  FastDiv fd_nstrip;  // output strips per row
  FastDiv fd_pstrips; // strips per plane of a several-plane block (Ho * strips per row)
};

constexpr int kStrip = 4;

template <int DT, int KH, int KW, int S>
__global__ __launch_bounds__(kThreads) void dw_kernel(const ConvArgs a, const DwPlan pl) {
  typedef typename Dw<DT>::T T;
  typedef typename Dw<DT>::A A;
  extern __shared__ __attribute__((aligned(16))) char dw_smem[];
  A* tile = (A*)dw_smem;                                   // [P][RIN][WP] (+ slack)
  const int tile_elems = pl.P * pl.RIN * pl.WP + 64;
  A* wts = tile + tile_elems;                              // [P][kH*kW]

  const int kH = KH ? KH : a.kH, kW = KW ? KW : a.kW;
  const int sh = S ? S : a.sh, sw = S ? S : a.sw;
  const int dh = KH ? 1 : a.dh, dw = KH ? 1 : a.dw;
  const int KK = kH * kW;
  const int C = a.C, H = a.H, W = a.W, Ho = a.Ho, Wo = a.Wo;
  const int nplanes = a.N * C;
  const int pl0 = blockIdx.x * pl.P;
  const int oh0 = blockIdx.y * pl.TH;
  const int th = min(pl.TH, Ho - oh0);
  const int np = min(pl.P, nplanes - pl0);
  const int ih_start = oh0 * sh - a.pt;                    // input row of LDS row 0
  const int rin = (th - 1) * sh + (kH - 1) * dh + 1;       // rows this block needs

  I8View q;
  A padv = (A)0;
  if constexpr (DT == DT_I8) {
    q.init(a.i8);
    padv = (A)q.xzp;
  }

  // weights of the block's channels
  const T* Wt = (const T*)a.Wt;
  for (int i = threadIdx.x; i < np * KK; i += kThreads) {
    const int pp = i / KK;
    const int c = (pl0 + pp) % C;
    wts[i] = widen<T, A>(Wt[c * KK + (i - pp * KK)]);
  }

  // halo cells: rows outside the image, and columns left/right of it
  for (int i = threadIdx.x; i < np * rin; i += kThreads) {
    const int pp = i / rin, r = i - (i / rin) * rin;
    const int ih = ih_start + r;
    A* row = tile + (pp * pl.RIN + r) * pl.WP;
    if ((unsigned)ih >= (unsigned)H) {
      for (int j = 0; j < pl.WP; ++j) row[j] = padv;
    } else {
      for (int j = 0; j < min(a.pl, pl.WP); ++j) row[j] = padv;
      for (int j = a.pl + W; j < pl.WP; ++j) row[j] = padv;
    }
  }

  // interior: the block's input is one contiguous span of X -- rows [r_lo,
  // r_hi) of one plane, or all rows of its np planes -- read as a flat array
  // with 16-byte loads (an unaligned head and the tail element-wise) and
  // scattered to (plane, row, column) of the LDS tile, every load of the
  // block in flight at once.
  const int r_lo = max(0, -ih_start), r_hi = min(rin, H - ih_start);
  const int wcopy = min(W, pl.WP - a.pl);                  // input columns used
  if (r_hi > r_lo && wcopy > 0) {
    const T* X = (const T*)a.X;
    constexpr int EPC = 16 / sizeof(T);
    const int nrow = r_hi - r_lo;
    const T* src0 = X + ((int64_t)pl0 * H + (ih_start + r_lo)) * (int64_t)W;
    A* dst0 = tile + r_lo * pl.WP + a.pl;
    // np > 1 (whole images, TH == Ho): the span is all H rows of each plane,
    // of which the first nrow are staged (a strided kernel may not reach the
    // last rows); np == 1: the span is the nrow staged rows
    const int span = np == 1 ? nrow * W : np * H * W;
    // element f of the span -> LDS cell (or -1 when its row or column is not needed)
    auto cell = [&](int f) {
      int pp = 0, rem = f;
      if (np > 1) {
        pp = fdiv(pl.fd_plane, f);
        rem = f - pp * H * W;
      }
      const int r = fdiv(pl.fd_w, rem);
      const int cc = rem - r * W;
      return (cc < wcopy && r < nrow) ? (pp * pl.RIN + r) * pl.WP + cc : -1;
    };
    const int head = min(span, (int)(((16 - (((uintptr_t)src0) & 15)) & 15) / sizeof(T)));
    const int nvec = (span - head) / EPC;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
      const int f0 = head + v * EPC;
      const u32x4_t raw = *(const u32x4_t*)(src0 + f0);
      T e[EPC];
      __builtin_memcpy(e, &raw, 16);
      // walk (plane, row, column) from the first element
      int pp = 0, rem = f0;
      if (np > 1) {
        pp = fdiv(pl.fd_plane, f0);
        rem = f0 - pp * H * W;
      }
      int r = fdiv(pl.fd_w, rem);
      int cc = rem - r * W;
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        if (cc < wcopy && r < nrow) dst0[(pp * pl.RIN + r) * pl.WP + cc] = widen<T, A>(e[j]);
        if (++cc == W) {
          cc = 0;
          if (++r == H) {            // next plane (np > 1 only: a one-plane span ends first)
            r = 0;
            ++pp;
          }
        }
      }
    }
    for (int f = threadIdx.x; f < head; f += kThreads) {
      const int d = cell(f);
      if (d >= 0) dst0[d] = widen<T, A>(src0[f]);
    }
    for (int f = head + nvec * EPC + threadIdx.x; f < span; f += kThreads) {
      const int d = cell(f);
      if (d >= 0) dst0[d] = widen<T, A>(src0[f]);
    }
  }
  __syncthreads();

  // compute: strips of kStrip outputs along a row
  const int nstrip = (Wo + kStrip - 1) / kStrip;
  const int per_plane = th * nstrip;
  const T* bias = (const T*)a.bias;
  for (int t = threadIdx.x; t < np * per_plane; t += kThreads) {
    const int pp = np > 1 ? fdiv(pl.fd_pstrips, t) : 0;   // (np > 1: th == Ho)
    const int rem = t - pp * per_plane;
    const int r = fdiv(pl.fd_nstrip, rem);
    const int ow0 = (rem - r * nstrip) * kStrip;
    const int64_t plane = pl0 + pp;
    const int c = (int)(plane % C);
    const A* wk = wts + pp * KK;
    A acc[kStrip];
    A init = (A)0;
    if constexpr (DT == DT_I8) init = q.bias[c];
#pragma unroll
    for (int o = 0; o < kStrip; ++o) acc[o] = init;

    if constexpr (KH > 0) {
      constexpr int WIN = (kStrip - 1) * S + KW;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const A* rp = tile + (pp * pl.RIN + r * S + kh) * pl.WP + ow0 * S;
        A win[WIN];
#pragma unroll
        for (int j = 0; j < WIN; ++j) win[j] = rp[j];
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
          const A wv = wk[kh * KW + kw];
#pragma unroll
          for (int o = 0; o < kStrip; ++o) acc[o] += win[o * S + kw] * wv;
        }
      }
    } else {
      for (int kh = 0; kh < kH; ++kh) {
        const A* rp = tile + (pp * pl.RIN + r * sh + kh * dh) * pl.WP + ow0 * sw;
        for (int kw = 0; kw < kW; ++kw) {
          const A wv = wk[kh * kW + kw];
#pragma unroll
          for (int o = 0; o < kStrip; ++o) acc[o] += rp[o * sw + kw * dw] * wv;
        }
      }
    }

    const int oh = oh0 + r;
    const int64_t ybase = (plane * Ho + oh) * (int64_t)Wo + ow0;
    if constexpr (DT == DT_I8) {
#pragma unroll
      for (int o = 0; o < kStrip; ++o) {
        if (ow0 + o < Wo) {
          if (a.out_dt == DT_I32) ((int32_t*)a.Y)[ybase + o] = acc[o];
          else ((int8_t*)a.Y)[ybase + o] = requant(acc[o], q.mult[c], q.yzp);
        }
      }
    } else {
      const float bv = bias ? to_f32(bias[c]) : 0.0f;
      with_act(a.act, [&](auto act_k) {
        constexpr int ACT = decltype(act_k)::value;
#pragma unroll
        for (int o = 0; o < kStrip; ++o) {
          if (ow0 + o < Wo) {
            const float v = act_c<ACT>(acc[o] + bv);
            if constexpr (DT == DT_BF16) ((uint16_t*)a.Y)[ybase + o] = f32_to_bf16(v);
            else ((float*)a.Y)[ybase + o] = v;
          }
        }
      });
    }
  }
}

constexpr int kLdsCap = 64 * 1024;

int lds_bytes(const DwPlan& p, int KK) {
  return (p.P * p.RIN * p.WP + 64 + p.P * KK) * 4;
}

DwPlan make_plan(const ConvArgs& a) {
  DwPlan p;
  const int nstrip = (a.Wo + kStrip - 1) / kStrip;
  p.fd_w = make_fastdiv((uint32_t)std::max(1, a.W));
  p.fd_plane = make_fastdiv((uint32_t)std::max(1, a.H * a.W));
  p.fd_nstrip = make_fastdiv((uint32_t)std::max(1, nstrip));
  p.fd_pstrips = make_fastdiv((uint32_t)std::max(1, a.Ho * nstrip));
  p.OWT = kStrip;
  p.WP = (a.Wo - 1) * a.sw + (a.kW - 1) * a.dw + 1 + kStrip * a.sw;   // + strip overrun
  const int KK = a.kH * a.kW;
  const int per_plane = a.Ho * a.Wo;
  auto rin = [&](int th) { return (th - 1) * a.sh + (a.kH - 1) * a.dh + 1; };
  // Outputs per block: sized so that a block stages about 4096 input pixels
  // (2048 for planes under 512 pixels, where more blocks hide the latency
  // better); a strided kernel reads sh*sw input pixels per output.
  int target = (a.H * a.W >= 512 ? 4096 : 2048) / std::max(1, a.sh * a.sw);
  if (const char* e = getenv("OX_DW_TARGET")) target = std::max(64, std::min(65536, atoi(e)));  // tuning override
  if (per_plane >= target / 2) {
    p.P = 1;
    p.TH = std::max(1, std::min(a.Ho, target / std::max(1, a.Wo)));
    p.RIN = rin(p.TH);
    while (p.TH > 1 && lds_bytes(p, KK) > kLdsCap) {
      --p.TH;
      p.RIN = rin(p.TH);
    }
  } else {
    p.TH = a.Ho;
    p.RIN = rin(p.TH);
    p.P = std::max(1, target / per_plane);
    while (p.P > 1 && lds_bytes(p, KK) > kLdsCap) --p.P;
  }
  return p;
}

template <int DT>
int launch_dt(const ConvArgs& a, hipStream_t s) {
  const DwPlan p = make_plan(a);
  const int KK = a.kH * a.kW;
  const int bytes = lds_bytes(p, KK);
  if (bytes > kLdsCap) return (int)hipErrorInvalidConfiguration;
  const int64_t nplanes = (int64_t)a.N * a.C;
  dim3 grid((unsigned)((nplanes + p.P - 1) / p.P), (a.Ho + p.TH - 1) / p.TH, 1);
  const bool d1 = a.dh == 1 && a.dw == 1;
  if (d1 && a.kH == 3 && a.kW == 3 && a.sh == 1 && a.sw == 1)
    hipLaunchKernelGGL((dw_kernel<DT, 3, 3, 1>), grid, dim3(kThreads), bytes, s, a, p);
  else if (d1 && a.kH == 3 && a.kW == 3 && a.sh == 2 && a.sw == 2)
    hipLaunchKernelGGL((dw_kernel<DT, 3, 3, 2>), grid, dim3(kThreads), bytes, s, a, p);
  else if (d1 && a.kH == 1 && a.kW == 9 && a.sh == 1 && a.sw == 1)
    hipLaunchKernelGGL((dw_kernel<DT, 1, 9, 1>), grid, dim3(kThreads), bytes, s, a, p);
  else
    hipLaunchKernelGGL((dw_kernel<DT, 0, 0, 0>), grid, dim3(kThreads), bytes, s, a, p);
  return (int)hipGetLastError();
}

}  // namespace

bool depthwise_fits(const ConvArgs& a) {
  const DwPlan p = make_plan(a);
  return lds_bytes(p, a.kH * a.kW) <= kLdsCap && (a.Ho + p.TH - 1) / p.TH <= 65535;
}

int launch_conv_depthwise(const ConvArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (a.dt) {
    case DT_F32: return launch_dt<DT_F32>(a, s);
    case DT_BF16: return launch_dt<DT_BF16>(a, s);
    case DT_I8: return launch_dt<DT_I8>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace ox
