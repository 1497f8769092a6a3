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
// (or 8) adjacent outputs of one row, reusing one window of LDS values per
// kernel row across the strip.  Common shapes (3x3 stride 1/2, 1x9 stride 1,
// dilation 1) are compiled with fixed loop bounds; any other geometry runs a
// generic variant of the same scheme.  For bf16 and int8 blocks of one plane
// a thread walks a run of consecutive rows instead, its taps in registers
// and its window of input rows sliding down (one or two new rows per step,
// read as 16-byte vectors).
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <type_traits>

#include "engine.hpp"

namespace ox {

namespace {

// T: element in HBM; A: accumulator; L: element of the LDS tile, four bytes
// (widened once, as it is staged, so the inner loop reads ready operands)
template <int DT> struct Dw;
template <> struct Dw<DT_F32> { typedef float T; typedef float A; typedef float L; };
template <> struct Dw<DT_BF16> { typedef uint16_t T; typedef float A; typedef float L; };
template <> struct Dw<DT_I8> { typedef int8_t T; typedef int A; typedef int L; };

template <typename T, typename A> __device__ __forceinline__ A widen(T v);
template <> __device__ __forceinline__ float widen<float, float>(float v) { return v; }
template <> __device__ __forceinline__ float widen<uint16_t, float>(uint16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ int widen<int8_t, int>(int8_t v) { return (int)v; }
template <> __device__ __forceinline__ uint16_t widen<uint16_t, uint16_t>(uint16_t v) { return v; }
template <> __device__ __forceinline__ int widen<int, int>(int v) { return v; }

struct DwPlan {
  int TH;     // output rows per block
  int P;      // planes per block
  int RIN;    // input rows staged per plane
  int WP;     // staged row width (input columns incl. left/right halo)
  int OWT;    // outputs per thread strip (4)
  FastDiv fd_w;       // input row length W
  FastDiv fd_plane;   // H*W: span of one input plane (blocks of several planes)
  FastDiv fd_nstrip;  // output strips per row
  FastDiv fd_ho;      // output rows Ho (rows of a several-plane block, plane-major)
  FastDiv fd_c;       // channels C (plane -> channel)
  FastDiv fd_kk;      // taps kH*kW
  bool slide;         // sliding-window strips (fixed shape, one plane per block)
};

// 16-byte loads per thread issued at once in the staging phase (about 96, 64
// and 48 bytes); a plan sizes its blocks to stay within them.
template <int DT> struct DwLoads;
template <> struct DwLoads<DT_F32> { static constexpr int V = 6; };
template <> struct DwLoads<DT_BF16> { static constexpr int V = 4; };
template <> struct DwLoads<DT_I8> { static constexpr int V = 3; };

// Outputs per thread strip: 4, or 8 where the row length wastes no more
// outputs that way (halving the per-strip index and store bookkeeping).  A
// strip is written in chunks of 4 (one 4-wide store where full and aligned).
constexpr int kChunk = 4;

template <int DT, int KH, int KW, int S, int ST, bool SLIDE, bool MAXP = false>
__global__ __launch_bounds__(kThreads) void dw_kernel(const ConvArgs a, const DwPlan pl) {
  static_assert(ST % kChunk == 0, "strips are whole store chunks");
  typedef typename Dw<DT>::T T;
  typedef typename Dw<DT>::A A;
  extern __shared__ __attribute__((aligned(16))) char dw_smem[];
  typedef typename Dw<DT>::L L;
  L* tile = (L*)dw_smem;                                   // [P][RIN][WP] (+ slack)
  const int tile_bytes = ((pl.P * pl.RIN * pl.WP + 64) * (int)sizeof(L) + 15) & ~15;
  A* wts = (A*)(dw_smem + tile_bytes);                     // [P][kH*kW]
  A* pbias = wts + pl.P * (KH ? KH * KW : a.kH * a.kW);    // [P] per-plane bias (fp32 / int32)
  double* pmult = (double*)(((uintptr_t)(pbias + pl.P) + 7) & ~(uintptr_t)7);  // [P] int8 multipliers

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
  L padv = (L)0;
  if constexpr (DT == DT_I8) {
    q.init(a.i8);
    padv = (L)q.xzp;
  }
  // an input element as staged: int8 in its int8 view (a uint8 byte with the
  // top bit flipped, u - 128), the float types widened
  auto wx = [&](T v) -> L {
    if constexpr (DT == DT_I8) return (L)(int8_t)((uint8_t)v ^ (uint8_t)q.xm);
    else return widen<T, L>(v);
  };
  // a weight as used: int8 minus its channel's zero point (Wt index i)
  auto ww = [&](T v, int i) -> A {
    if constexpr (DT == DT_I8) return (A)v - (q.wz ? q.wzp[i / KK] : 0);
    else return widen<T, A>(v);
  };
  if constexpr (MAXP) padv = (L)-INFINITY;      // MaxPool: padding never wins

  // Every global load of the staging phase is issued before the first wait:
  // the interior as 16-byte vectors into registers (at most kLoads per
  // thread; a plan keeps the span within that, and a loop after the first
  // wave of loads takes any remainder), the span's unaligned head and tail
  // elements, and up to two weights per thread.  The halo is filled while the
  // loads are in flight, then everything is written to LDS.
  const int r_lo = max(0, -ih_start), r_hi = min(rin, H - ih_start);
  const bool any = r_hi > r_lo;
  const int nrow = any ? r_hi - r_lo : 0;
  const T* src0 = (const T*)a.X + ((int64_t)pl0 * H + (ih_start + r_lo)) * (int64_t)W;
  L* dst0 = tile + r_lo * pl.WP + a.pl;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int NV = DwLoads<DT>::V;
  // the block's input is one contiguous span of X: rows [r_lo, r_hi) of one
  // plane, or all H rows of each of its np planes (whole images, TH == Ho),
  // of which the first nrow are staged (a strided kernel may not reach the
  // last rows)
  const int span = !any ? 0 : (np == 1 ? nrow * W : np * H * W);
  const int head = min(span, (int)(((16 - (((uintptr_t)src0) & 15)) & 15) / sizeof(T)));
  const int nvec = (span - head) / EPC;
  const int tail0 = head + nvec * EPC;
  const int tid = threadIdx.x;
  const T* Wt = (const T*)a.Wt;
  const int nw = np * KK;
  auto chan = [&](int plane) { return plane - fdiv(pl.fd_c, plane) * C; };
  auto widx = [&](int i) {                                 // weight i of the block -> index in Wt
    const int pp = KH ? i / KK : fdiv(pl.fd_kk, i);
    return chan(pl0 + pp) * KK + (i - pp * KK);
  };
  const int wi0 = widx(min(tid, nw - 1)), wi1 = widx(min(tid + kThreads, nw - 1));
  const int cb = chan(pl0 + min(tid, np - 1));             // channel of this thread's plane value
  // (every thread issues all NV vector loads, lanes past the end re-reading
  // the last vector, so that no load is predicated)
  const int ntail = span - tail0;
  u32x4_t buf[NV];
  if (nvec > 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      buf[i] = *(const u32x4_t*)(src0 + head + min(tid + i * kThreads, nvec - 1) * EPC);
  }
  // head and tail elements (a block with an empty span reads a weight instead)
  // (MaxPool has no weights: nothing is read in their place)
  const T he = span > 0 ? src0[min(tid, span - 1)] : (MAXP ? (T)0 : Wt[wi0]);
  const T te = span > 0 ? src0[min(tail0 + tid, span - 1)] : (MAXP ? (T)0 : Wt[wi0]);
  const T w0 = MAXP ? (T)0 : Wt[wi0], w1 = MAXP ? (T)0 : Wt[wi1];
  // the bias of plane tid (and its int8 multiplier)
  A b0 = (A)0;
  double m0 = 0.0;
  const T* bias = (const T*)a.bias;
  // (int8 with weight zero points: the weights are used as w - w_zp, so the
  // folded bias, bias - x_zp * sum w, gains x_zp * kH*kW * w_zp)
  if constexpr (DT == DT_I8) {
    b0 = q.bias[cb] + (q.wz ? q.xzp * KK * q.wzp[cb] : 0);
    m0 = q.mult[cb];
  } else {
    if (bias) b0 = widen<T, A>(bias[cb]);
  }

  // halo cells: rows outside the image, and columns left/right of it
  for (int i = tid; i < np * rin; i += kThreads) {
    const int pp = i / rin, r = i - (i / rin) * rin;
    const int ih = ih_start + r;
    L* row = tile + (pp * pl.RIN + r) * pl.WP;
    if ((unsigned)ih >= (unsigned)H) {
      for (int j = 0; j < pl.WP; ++j) row[j] = padv;
    } else {
      for (int j = 0; j < min(a.pl, pl.WP); ++j) row[j] = padv;
      for (int j = a.pl + W; j < pl.WP; ++j) row[j] = padv;
    }
  }

  if (tid < nw) wts[tid] = ww(w0, wi0);
  if (tid + kThreads < nw) wts[tid + kThreads] = ww(w1, wi1);
  if constexpr (!MAXP)
    for (int i = tid + 2 * kThreads; i < nw; i += kThreads) {
      const int wi = widx(i);
      wts[i] = ww(Wt[wi], wi);
    }
  auto plane_vals = [&](int i, A bv, double mv) {
    pbias[i] = bv;
    if constexpr (DT == DT_I8) pmult[i] = mv;
  };
  if (tid < np) plane_vals(tid, b0, m0);
  for (int i = tid + kThreads; i < np; i += kThreads) {
    const int c = chan(pl0 + i);
    if constexpr (DT == DT_I8) plane_vals(i, q.bias[c] + (q.wz ? q.xzp * KK * q.wzp[c] : 0), q.mult[c]);
    else plane_vals(i, bias ? widen<T, A>(bias[c]) : (A)0, 0.0);
  }

  // element f of the span -> LDS cell (or -1 when its row or column is not needed)
  auto cell = [&](int f) {
    int pp = 0, rem = f;
    if (np > 1) {
      pp = fdiv(pl.fd_plane, f);
      rem = f - pp * H * W;
    }
    const int r = fdiv(pl.fd_w, rem);
    const int cc = rem - r * W;
    return (pp * pl.RIN + r) * pl.WP + cc;
  };
  // the EPC elements of vector v.  Every element of the span has a cell (the
  // plan makes rows at least pl + W wide and, for several-plane blocks, keeps
  // all H rows of each plane), so nothing is predicated: a vector that stays
  // in one row goes to consecutive cells; one that reaches the end of its row
  // (W >= EPC: at most once) continues at column 0 of the next row, which may
  // be the first row of the next plane; narrower rows walk element by element.
  auto scatter = [&](int v, const u32x4_t& raw) {
    const int f0 = head + v * EPC;
    T e[EPC];
    __builtin_memcpy(e, &raw, 16);
    int pp = 0, rem = f0;
    if (np > 1) {
      pp = fdiv(pl.fd_plane, f0);
      rem = f0 - pp * H * W;
    }
    int r = fdiv(pl.fd_w, rem);
    int cc = rem - r * W;
    L* d = dst0 + (pp * pl.RIN + r) * pl.WP + cc;
    if (W >= EPC) {
      const int k = W - cc;                                // cells left in this row
      if (k >= EPC) {
#pragma unroll
        for (int j = 0; j < EPC; ++j) d[j] = wx(e[j]);
      } else {
        const int gap = (pl.WP - W) + (r + 1 == H ? (pl.RIN - H) * pl.WP : 0);
#pragma unroll
        for (int j = 0; j < EPC; ++j) d[j + (j >= k ? gap : 0)] = wx(e[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPC; ++j) {
        dst0[(pp * pl.RIN + r) * pl.WP + cc] = wx(e[j]);
        if (++cc == W) {
          cc = 0;
          if (++r == H) {          // next plane (np > 1 only: a one-plane span ends first)
            r = 0;
            ++pp;
          }
        }
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = tid + i * kThreads;
    if (v < nvec) scatter(v, buf[i]);
  }
  for (int v = tid + NV * kThreads; v < nvec; v += kThreads)
    scatter(v, *(const u32x4_t*)(src0 + head + v * EPC));
  if (tid < head) dst0[cell(tid)] = wx(he);
  if (tid < ntail) dst0[cell(tail0 + tid)] = wx(te);
  __syncthreads();

  // compute: strips of ST outputs along a row.  The block's output rows are
  // numbered plane-major (q = pp * th + r).
  const int nstrip = (Wo + ST - 1) / ST;
  const int nq = np * th;
  const int64_t yblock = ((int64_t)pl0 * Ho + oh0) * Wo;  // output offset of (plane pl0, row oh0)
  // every strip full and every 4-output chunk aligned for one vector store
  // (rows a multiple of the strip, Y aligned): stores need no per-chunk test
  constexpr int osize = DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1;
  const int ysize = (DT == DT_I8 && a.out_dt == DT_I32) ? 4 : osize;
  const bool fast = Wo % ST == 0 && ((uintptr_t)a.Y % (uintptr_t)(4 * ysize)) == 0;

  // each chunk of 4 outputs that is full and aligned is written with one
  // 4x-wide store (whole cache lines per wave instead of partial lines)
  auto store_strip = [&](int pp, int r, int ow0, const A (&acc)[ST], auto act_k) {
    constexpr int ACT = decltype(act_k)::value;
    const int yoff = (pp * Ho + r) * Wo + ow0;             // within the block's output span
    double mv = 0.0;
    if constexpr (DT == DT_I8) mv = pmult[pp];
#pragma unroll
    for (int c4 = 0; c4 < ST; c4 += kChunk) {
      const A* ac = acc + c4;
      const int o0 = ow0 + c4;
      const bool full = fast || o0 + kChunk <= Wo;
      if constexpr (DT == DT_I8) {
        if (a.out_dt == DT_I32) {
          int32_t* yp = (int32_t*)a.Y + yblock + yoff + c4;
          if (fast || (full && ((uintptr_t)yp & 15) == 0)) {
            *(i32x4_t*)yp = i32x4_t{ac[0], ac[1], ac[2], ac[3]};
          } else {
#pragma unroll
            for (int o = 0; o < kChunk; ++o)
              if (o0 + o < Wo) yp[o] = ac[o];
          }
        } else {
          int8_t* yp = (int8_t*)a.Y + yblock + yoff + c4;
          int8_t v[kChunk];
#pragma unroll
          for (int o = 0; o < kChunk; ++o) v[o] = (int8_t)(requant(ac[o], mv, q.yzp) ^ q.ym);
          if (fast || (full && ((uintptr_t)yp & 3) == 0)) {
            uint32_t w;
            __builtin_memcpy(&w, v, 4);
            *(uint32_t*)yp = w;
          } else {
#pragma unroll
            for (int o = 0; o < kChunk; ++o)
              if (o0 + o < Wo) yp[o] = v[o];
          }
        }
      } else {
        float v[kChunk];
#pragma unroll
        for (int o = 0; o < kChunk; ++o) v[o] = act_c<ACT>(ac[o]);
        if constexpr (DT == DT_BF16) {
          uint16_t* yp = (uint16_t*)a.Y + yblock + yoff + c4;
          if (fast || (full && ((uintptr_t)yp & 7) == 0)) {
            *(u32x2_t*)yp = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
#pragma unroll
            for (int o = 0; o < kChunk; ++o)
              if (o0 + o < Wo) yp[o] = f32_to_bf16(v[o]);
          }
        } else {
          float* yp = (float*)a.Y + yblock + yoff + c4;
          if (fast || (full && ((uintptr_t)yp & 15) == 0)) {
            *(f32x4_t*)yp = f32x4_t{v[0], v[1], v[2], v[3]};
          } else {
#pragma unroll
            for (int o = 0; o < kChunk; ++o)
              if (o0 + o < Wo) yp[o] = v[o];
          }
        }
      }
    }
  };

  // any geometry: one strip, every tap read from LDS
  auto strip = [&](int pp, int r, int ow0, auto act_k) {
    const A* wk = wts + pp * KK;
    A acc[ST];
    const A init = MAXP ? (A)-INFINITY : pbias[pp];       // the bias seeds the accumulators
#pragma unroll
    for (int o = 0; o < ST; ++o) acc[o] = init;
    for (int kh = 0; kh < kH; ++kh) {
      const L* rp = tile + (pp * pl.RIN + r * sh + kh * dh) * pl.WP + ow0 * sw;
      for (int kw = 0; kw < kW; ++kw) {
        const A wv = wk[kh * kW + kw];
#pragma unroll
        for (int o = 0; o < ST; ++o) {
          if constexpr (MAXP) acc[o] = fmaxf(acc[o], widen<L, A>(rp[o * sw + kw * dw]));
          else acc[o] += widen<L, A>(rp[o * sw + kw * dw]) * wv;
        }
      }
    }
    store_strip(pp, r, ow0, acc, act_k);
  };

  // row q of the block -> (plane, row); several planes only with th == Ho
  auto row_of = [&](int qq, int& pp, int& r) {
    pp = np > 1 ? fdiv(pl.fd_ho, qq) : 0;
    r = qq - pp * Ho;
  };

  // Fixed shapes: a thread owns one strip column and a run of consecutive
  // output rows of it.  Its taps stay in registers for the plane, and the
  // input rows form a window that slides down: a stride-1 step reads one new
  // row of the window, a stride-2 step two (the window's rows rotate through
  // KH register slots, the loop unrolled by KH so that the rotation is known
  // at compile time).  Rows are read as 16-byte vectors (the plan makes the
  // staged row pitch a multiple of 4 elements and strips start at multiples
  // of 4 elements).
  auto run_fixed = [&](auto act_k) {
    constexpr int WIN = (ST - 1) * S + KW;                 // input columns of a strip
    constexpr int WV = WIN > 0 ? (WIN + 3) / 4 : 1;        // 16-byte reads per window row
    constexpr int NSL = KH > 0 ? KH : 1;                   // register slots of window rows
    const int tpc = kThreads / nstrip;                     // runs per strip column
    const int rr = (nq + tpc - 1) / tpc;                   // rows per run
    const int ri = fdiv(pl.fd_nstrip, tid);
    const int ow0 = (tid - ri * nstrip) * ST;
    const int qa = ri * rr, qb = min(nq, qa + rr);
    if (ri >= tpc || qa >= qb) return;
    int pp, r;
    row_of(qa, pp, r);
    A wv[KK];
    A init = (A)0;
    L win[NSL][WV * 4];
    auto read_row = [&](L (&dst)[WV * 4], int row) {
      const L* rp = tile + (pp * pl.RIN + row) * pl.WP + ow0 * S;
      typedef L L4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int j = 0; j < WV; ++j) {
        const L4 v = *(const L4*)(rp + 4 * j);
        dst[4 * j] = v[0];
        dst[4 * j + 1] = v[1];
        dst[4 * j + 2] = v[2];
        dst[4 * j + 3] = v[3];
      }
    };
    auto step = [&](auto PHc, bool refill) {
      constexpr int PH = decltype(PHc)::value;
      if (refill) {
#pragma unroll
        for (int k = 0; k < KK; ++k) wv[k] = wts[pp * KK + k];
        init = MAXP ? (A)-INFINITY : pbias[pp];
        static_for<KH>([&](auto KHc) {
          constexpr int kh = decltype(KHc)::value;
          read_row(win[(kh + S * PH) % NSL], r * S + kh);
        });
      } else {
        static_for<KH>([&](auto KHc) {
          constexpr int kh = decltype(KHc)::value;
          if constexpr (kh >= KH - S || KH <= S) read_row(win[(kh + S * PH) % NSL], r * S + kh);
        });
      }
      A acc[ST];
#pragma unroll
      for (int o = 0; o < ST; ++o) acc[o] = init;
      static_for<KH>([&](auto KHc) {
        constexpr int kh = decltype(KHc)::value;
        const L* w = win[(kh + S * PH) % NSL];
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
          for (int o = 0; o < ST; ++o) {
            if constexpr (MAXP) acc[o] = fmaxf(acc[o], widen<L, A>(w[o * S + kw]));
            else acc[o] += widen<L, A>(w[o * S + kw]) * wv[kh * KW + kw];
          }
      });
      store_strip(pp, r, ow0, acc, act_k);
      if (++r == Ho) {                                     // next plane (several-plane blocks)
        r = 0;
        ++pp;
      }
    };
    for (int qq = qa; qq < qb; qq += NSL) {
      static_for<NSL>([&](auto PHc) {
        constexpr int PH = decltype(PHc)::value;
        if (qq + PH < qb) step(PHc, qq + PH == qa || (np > 1 && r == 0));
      });
    }
  };

  auto run = [&](auto act_k) {
    if constexpr (SLIDE) {
      run_fixed(act_k);     // (the plan takes SLIDE only where nstrip <= kThreads)
      return;
    }
    if (nstrip <= kThreads) {
      const int rpp = kThreads / nstrip;                   // rows per pass
      const int q0 = fdiv(pl.fd_nstrip, tid);
      const int ow0 = (tid - q0 * nstrip) * ST;
      if (q0 < rpp) {
        for (int qq = q0; qq < nq; qq += rpp) {
          int pp, r;
          row_of(qq, pp, r);
          strip(pp, r, ow0, act_k);
        }
      }
    } else {
      for (int t = tid; t < nq * nstrip; t += kThreads) {
        const int qq = fdiv(pl.fd_nstrip, t);
        int pp, r;
        row_of(qq, pp, r);
        strip(pp, r, (t - qq * nstrip) * ST, act_k);
      }
    }
  };
  if constexpr (DT == DT_I8) run(std::integral_constant<int, ACT_NONE>{});
  else with_act(a.act, run);
}

constexpr int kLdsCap = 64 * 1024;

// the tile (4-byte elements, 16-byte rounded), the fp32/int32 weights, the
// per-plane bias and (int8) the per-plane fp64 multipliers
int lds_bytes(const DwPlan& p, int KK) {
  return (((p.P * p.RIN * p.WP + 64) * 4 + 15) & ~15) + p.P * KK * 4 + p.P * 4 + 8 + p.P * 8;
}

// the fixed-shape kernels (3x3 stride 1 or 2, 1x9; dilation 1)
bool fixed_shape(const ConvArgs& a) {
  const bool d1 = a.dh == 1 && a.dw == 1;
  return d1 && ((a.kH == 3 && a.kW == 3 && a.sh == a.sw && (a.sh == 1 || a.sh == 2)) ||
                (a.kH == 1 && a.kW == 9 && a.sh == 1 && a.sw == 1));
}

int strip_width(const ConvArgs& a) {
  // (a stride-2 strip of 8 needs a 17-wide window; on short rows the
  // block's few strips would spread unevenly over its threads)
  if (!fixed_shape(a) || a.sh != 1 || a.Wo < 32) return 4;
  const int w4 = (a.Wo + 3) / 4 * 4, w8 = (a.Wo + 7) / 8 * 8;
  return w8 <= w4 ? 8 : 4;
}

DwPlan make_plan(const ConvArgs& a) {
  DwPlan p;
  p.OWT = strip_width(a);
  const int nstrip = (a.Wo + p.OWT - 1) / p.OWT;
  p.fd_w = make_fastdiv((uint32_t)std::max(1, a.W));
  p.fd_plane = make_fastdiv((uint32_t)std::max(1, a.H * a.W));
  p.fd_nstrip = make_fastdiv((uint32_t)std::max(1, nstrip));
  p.fd_ho = make_fastdiv((uint32_t)std::max(1, a.Ho));
  p.fd_c = make_fastdiv((uint32_t)std::max(1, a.C));
  p.fd_kk = make_fastdiv((uint32_t)std::max(1, a.kH * a.kW));
  // staged row: left halo, every input column (a strided kernel may not read
  // the last ones, but the staging copies whole rows), right halo and the
  // overrun of the last strip
  p.WP = std::max((a.Wo - 1) * a.sw + (a.kW - 1) * a.dw + 1 + p.OWT * a.sw, a.pl + a.W);
  const int KK = a.kH * a.kW;
  const int per_plane = a.Ho * a.Wo;
  auto rin = [&](int th) { return (th - 1) * a.sh + (a.kH - 1) * a.dh + 1; };
  // Outputs per block: a block stages about 4096 input pixels (2048 on
  // planes under 512 pixels, where more, smaller blocks balance better); a
  // strided kernel reads sh*sw input pixels per output, but on large planes
  // (2048+ pixels) a strided block does best with twice that share.
  const int sa = std::max(1, a.sh * a.sw);
  int target = (a.H * a.W >= 512 ? 4096 : 2048) / (sa > 1 && a.H * a.W >= 2048 ? std::max(1, sa / 2) : sa);
  if (const char* e = getenv("OX_DW_TARGET")) target = std::max(64, std::min(65536, atoi(e)));  // tuning override
  // one plane per block (a band of its rows), bf16 or int8: strips slide
  // down a run of rows, reading the staged rows as 16-byte vectors (row
  // pitch a multiple of 4 elements).  Blocks of several small planes keep
  // the leaner row-stride kernel: their runs would cross planes every few
  // rows, and the window's registers would cost them occupancy.  (Measured
  // on the MobileNetV2 layers at batch 64: -10..-17% on the three
  // single-plane bf16 layers; no gain in fp32, whose layers move twice the
  // bytes per output.)
  p.slide = fixed_shape(a) && a.dt != DT_F32 && per_plane >= target / 2 && nstrip <= kThreads;
  if (p.slide) p.WP = (p.WP + 3) & ~3;
  // input elements the staging phase's first wave of loads covers
  const int esize = a.dt == DT_F32 ? 4 : a.dt == DT_BF16 ? 2 : 1;
  const int64_t cap = (int64_t)(a.dt == DT_F32 ? DwLoads<DT_F32>::V
                                : a.dt == DT_BF16 ? DwLoads<DT_BF16>::V : DwLoads<DT_I8>::V) *
                      kThreads * (16 / esize);
  if (per_plane >= target / 2) {
    p.P = 1;
    p.TH = std::max(1, std::min(a.Ho, target / std::max(1, a.Wo)));
    p.RIN = rin(p.TH);
    while (p.TH > 1 && (lds_bytes(p, KK) > kLdsCap || (int64_t)p.RIN * a.W > cap)) {
      --p.TH;
      p.RIN = rin(p.TH);
    }
    // equal bands: the fewest bands of at most TH rows, with their rows spread evenly
    const int nb = (a.Ho + p.TH - 1) / p.TH;
    p.TH = (a.Ho + nb - 1) / nb;
    p.RIN = rin(p.TH);
  } else {
    p.TH = a.Ho;
    p.RIN = std::max(rin(p.TH), a.pt + a.H);               // whole planes are staged
    p.P = std::max(1, target / per_plane);
    while (p.P > 1 && (lds_bytes(p, KK) > kLdsCap || (int64_t)p.P * a.H * a.W > cap)) --p.P;
  }
  return p;
}

template <int DT, bool MAXP = false>
int launch_dt(const ConvArgs& a, hipStream_t s) {
  const DwPlan p = make_plan(a);
  const int KK = a.kH * a.kW;
  const int bytes = lds_bytes(p, KK);
  if (bytes > kLdsCap) return (int)hipErrorInvalidConfiguration;
  const int64_t nplanes = (int64_t)a.N * a.C;
  dim3 grid((unsigned)((nplanes + p.P - 1) / p.P), (a.Ho + p.TH - 1) / p.TH, 1);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kThreads), bytes, s, a, p); };
  const bool w8 = p.OWT == 8;
  auto go2 = [&](auto slide_k, auto plain_k) { p.slide ? go(slide_k) : go(plain_k); };
  if (!fixed_shape(a))
    go(dw_kernel<DT, 0, 0, 0, 4, false, MAXP>);
  else if (a.kH == 1)
    w8 ? go2(dw_kernel<DT, 1, 9, 1, 8, true, MAXP>, dw_kernel<DT, 1, 9, 1, 8, false, MAXP>)
       : go2(dw_kernel<DT, 1, 9, 1, 4, true, MAXP>, dw_kernel<DT, 1, 9, 1, 4, false, MAXP>);
  else if (a.sh == 1)
    w8 ? go2(dw_kernel<DT, 3, 3, 1, 8, true, MAXP>, dw_kernel<DT, 3, 3, 1, 8, false, MAXP>)
       : go2(dw_kernel<DT, 3, 3, 1, 4, true, MAXP>, dw_kernel<DT, 3, 3, 1, 4, false, MAXP>);
  else
    w8 ? go2(dw_kernel<DT, 3, 3, 2, 8, true, MAXP>, dw_kernel<DT, 3, 3, 2, 8, false, MAXP>)
       : go2(dw_kernel<DT, 3, 3, 2, 4, true, MAXP>, dw_kernel<DT, 3, 3, 2, 4, false, MAXP>);
  return (int)hipGetLastError();
}

}  // namespace

bool depthwise_fits(const ConvArgs& a) {
  const DwPlan p = make_plan(a);
  return lds_bytes(p, a.kH * a.kW) <= kLdsCap && (a.Ho + p.TH - 1) / p.TH <= 65535;
}

// MaxPool through the same staged-band kernel: the window is the depthwise
// window, -inf fills the halo and the taps are combined with max (no
// weights, no bias, no activation)
int launch_maxpool_dw(const ConvArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (a.dt) {
    case DT_F32: return launch_dt<DT_F32, true>(a, s);
    case DT_BF16: return launch_dt<DT_BF16, true>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
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
